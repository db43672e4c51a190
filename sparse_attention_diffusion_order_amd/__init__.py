"""Python binding of libllsa.so (MI355X / gfx950 Log-linear Sparse Attention).

Argument marshalling only: every step of the path runs in the HIP kernels of
libllsa.so.  The C entry points are exposed under the same names
(llsa_forward, llsa_backward, llsa_zorder, ...) and accept torch tensors (their
device pointers are passed) or raw integer addresses.  `stream=None` means
torch's current stream.  A nonzero return code raises LlsaError.

The library must have been built in-tree (sparse_attention_diffusion_order_amd/
libllsa.so, see build.py); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "LlsaError", "F32", "BF16", "NO_ENRICH", "ENRICH_COARSE", "SIZE_BIAS", "ENRICH_COMPLEMENT", "CAUSAL", "PART_POOL", "PART_SELECT", "PART_ATTN",
    "PART_TRANSPOSE", "PART_DQ", "PART_ENRICH", "PART_DKDV", "library_path", "load", "exported_names",
    "llsa_workspace_bytes", "llsa_workspace_layout", "llsa_zorder", "llsa_grid_order",
    "llsa_forward",
    "llsa_backward", "llsa_forward_part", "llsa_backward_part", "llsa_strerror",
    "llsa_workspace_bytes_lk", "llsa_workspace_layout_lk", "llsa_forward_lk", "llsa_backward_lk",
    "llsa_forward_noalloc", "llsa_forward_grid", "NOALLOC_SCRATCH_BYTES", "forward", "forward_grid",
    "backward", "zorder", "grid_order",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libllsa.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "llsa.h")

F32, BF16 = 0, 1
NO_ENRICH = 1
ENRICH_COARSE = 2
SIZE_BIAS = 4
ENRICH_COMPLEMENT = 8
CAUSAL = 16
PART_POOL, PART_SELECT, PART_ATTN = 0, 1, 2
PART_TRANSPOSE, PART_DQ, PART_DKDV, PART_ENRICH = 3, 4, 5, 6
MAX_LEVELS = 6
NOALLOC_SCRATCH_BYTES = 64 << 20  # LLSA_NOALLOC_SCRATCH_BYTES

_lib = None


class LlsaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %d (%s)" % (where, code, llsa_strerror(code)))


class WsLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t * MAX_LEVELS)
                for name in ("qbar", "kbar", "vbar", "idx", "rowptr", "col")] + \
               [("delta", ctypes.c_size_t), ("total", ctypes.c_size_t)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libllsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libllsa.so is not built (run sparse_attention_diffusion_order_amd/"
                          "build.py or __graft_entry__.build()); there is no fallback")
    lib = ctypes.CDLL(_LIB_PATH)
    I, P, U, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_uint, ctypes.c_size_t
    shape = [I] * 8  # B H N d block_size topk levels dtype
    lib.llsa_workspace_bytes.argtypes = shape
    lib.llsa_workspace_bytes.restype = S
    lib.llsa_workspace_layout.argtypes = shape + [ctypes.POINTER(WsLayout)]
    lib.llsa_workspace_layout.restype = I
    lib.llsa_zorder.argtypes = [P, P, ctypes.c_longlong, I, I, I, P]
    lib.llsa_zorder.restype = I
    lib.llsa_grid_order.argtypes = [P, P, ctypes.c_longlong, I, I, I, I, I, P]
    lib.llsa_grid_order.restype = I
    fwd = [P] * 5 + shape + [U, P, S, P]
    bwd = [P] * 9 + shape + [U, P, S, P]
    lib.llsa_forward.argtypes = fwd
    lib.llsa_forward.restype = I
    lib.llsa_backward.argtypes = bwd
    lib.llsa_backward.restype = I
    lib.llsa_forward_part.argtypes = [I] + fwd
    lib.llsa_forward_part.restype = I
    lib.llsa_backward_part.argtypes = [I] + bwd
    lib.llsa_backward_part.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lk = [I] * 5 + [IP, I, I]  # B H N d block_size topk[] levels dtype
    lib.llsa_workspace_bytes_lk.argtypes = lk
    lib.llsa_workspace_bytes_lk.restype = S
    lib.llsa_workspace_layout_lk.argtypes = lk + [ctypes.POINTER(WsLayout)]
    lib.llsa_workspace_layout_lk.restype = I
    lib.llsa_forward_lk.argtypes = [P] * 5 + lk + [U, P, S, P]
    lib.llsa_forward_lk.restype = I
    lib.llsa_backward_lk.argtypes = [P] * 9 + lk + [U, P, S, P]
    lib.llsa_backward_lk.restype = I
    lib.llsa_forward_noalloc.argtypes = [P] * 5 + shape + [U, P]
    lib.llsa_forward_noalloc.restype = I
    lib.llsa_forward_grid.argtypes = [P] * 8 + [I] * 10 + [U, P, S, P]
    lib.llsa_forward_grid.restype = I
    lib.llsa_strerror.argtypes = [I]
    lib.llsa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def exported_names():
    """Function names declared in include/llsa.h."""
    txt = open(_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(llsa_\w+)\s*\(", txt,
                                 flags=re.M)))


def _ptr(x):
    """Device address of a tensor (or a raw integer address, passed as is).
    A tensor that is not in GPU memory is refused: its host address would
    reach the kernels."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("libllsa takes device memory; got a tensor on %s" % x.device)
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != 0:
        raise LlsaError(rc, where)


def llsa_strerror(code: int) -> str:
    return load().llsa_strerror(code).decode()


def llsa_workspace_bytes(B, H, N, d, block_size, topk, levels, dtype) -> int:
    return int(load().llsa_workspace_bytes(B, H, N, d, block_size, topk, levels, dtype))


def llsa_workspace_layout(B, H, N, d, block_size, topk, levels, dtype) -> dict:
    lay = WsLayout()
    _check(load().llsa_workspace_layout(B, H, N, d, block_size, topk, levels, dtype,
                                        ctypes.byref(lay)), "llsa_workspace_layout")
    out = {name: list(getattr(lay, name))[:levels]
           for name in ("qbar", "kbar", "vbar", "idx", "rowptr", "col")}
    out["delta"], out["total"] = lay.delta, lay.total
    return out


def llsa_zorder(src, dst, outer, side, inner_bytes, inverse=0, stream=None):
    _check(load().llsa_zorder(_ptr(src), _ptr(dst), outer, side, inner_bytes, int(inverse),
                              _stream(stream)), "llsa_zorder")


def llsa_grid_order(src, dst, outer, frames, height, width, inner_bytes, inverse=0, stream=None):
    _check(load().llsa_grid_order(_ptr(src), _ptr(dst), outer, frames, height, width,
                                  inner_bytes, int(inverse), _stream(stream)), "llsa_grid_order")


def _karr(topk):
    """a per-level top-k sequence (level 1 first) as a C int array"""
    ks = [int(x) for x in topk]
    return (ctypes.c_int * max(1, len(ks)))(*ks)


def llsa_workspace_bytes_lk(B, H, N, d, block_size, topk, levels, dtype) -> int:
    return int(load().llsa_workspace_bytes_lk(B, H, N, d, block_size, _karr(topk), levels,
                                              dtype))


def llsa_workspace_layout_lk(B, H, N, d, block_size, topk, levels, dtype) -> dict:
    lay = WsLayout()
    _check(load().llsa_workspace_layout_lk(B, H, N, d, block_size, _karr(topk), levels, dtype,
                                           ctypes.byref(lay)), "llsa_workspace_layout_lk")
    out = {name: list(getattr(lay, name))[:levels]
           for name in ("qbar", "kbar", "vbar", "idx", "rowptr", "col")}
    out["delta"], out["total"] = lay.delta, lay.total
    return out


def llsa_forward_lk(q, k, v, out, lse, B, H, N, d, block_size, topk, levels, dtype, flags,
                    workspace, ws_bytes, stream=None):
    _check(load().llsa_forward_lk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                                  block_size, _karr(topk), levels, dtype, flags,
                                  _ptr(workspace), ws_bytes, _stream(stream)), "llsa_forward_lk")


def llsa_backward_lk(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, block_size, topk, levels,
                     dtype, flags, workspace, ws_bytes, stream=None):
    _check(load().llsa_backward_lk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, block_size,
                                   _karr(topk), levels, dtype, flags, _ptr(workspace),
                                   ws_bytes, _stream(stream)), "llsa_backward_lk")


def llsa_forward(q, k, v, out, lse, B, H, N, d, block_size, topk, levels, dtype, flags,
                 workspace, ws_bytes, stream=None):
    _check(load().llsa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                               block_size, topk, levels, dtype, flags, _ptr(workspace),
                               ws_bytes, _stream(stream)), "llsa_forward")


def llsa_backward(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, block_size, topk, levels,
                  dtype, flags, workspace, ws_bytes, stream=None):
    _check(load().llsa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, block_size, topk,
                                levels, dtype, flags, _ptr(workspace), ws_bytes,
                                _stream(stream)), "llsa_backward")


def llsa_forward_noalloc(q, k, v, out, lse, B, H, N, d, block_size, topk, levels, dtype, flags,
                         stream=None):
    _check(load().llsa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N,
                                       d, block_size, topk, levels, dtype, flags,
                                       _stream(stream)), "llsa_forward_noalloc")


def llsa_forward_grid(q_raster, k_raster, v_raster, q, k, v, out, lse, B, H, frames, height,
                      width, d, block_size, topk, levels, dtype, flags, workspace, ws_bytes,
                      stream=None):
    _check(load().llsa_forward_grid(_ptr(q_raster), _ptr(k_raster), _ptr(v_raster), _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, frames, height,
                                    width, d, block_size, topk, levels, dtype, flags,
                                    _ptr(workspace), ws_bytes, _stream(stream)),
           "llsa_forward_grid")


def llsa_forward_part(part, q, k, v, out, lse, B, H, N, d, block_size, topk, levels, dtype,
                      flags, workspace, ws_bytes, stream=None):
    _check(load().llsa_forward_part(part, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B,
                                    H, N, d, block_size, topk, levels, dtype, flags,
                                    _ptr(workspace), ws_bytes, _stream(stream)),
           "llsa_forward_part")


def llsa_backward_part(part, q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, block_size, topk,
                       levels, dtype, flags, workspace, ws_bytes, stream=None):
    _check(load().llsa_backward_part(part, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                     block_size, topk, levels, dtype, flags, _ptr(workspace),
                                     ws_bytes, _stream(stream)), "llsa_backward_part")


# ---------------------------------------------------------------- helpers
# Convenience wrappers over the entry points above for torch tensors shaped
# [B, H, N, d]; they allocate outputs and the workspace with torch.

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _check_tensors(named, shape, dtype, device):
    """every tensor contiguous, on `device` (a GPU), with `shape` and `dtype`"""
    for name, t in named:
        if not getattr(t, "is_cuda", False) or t.device != device:
            raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
        if t.dtype != dtype or tuple(t.shape) != tuple(shape):
            raise ValueError("%s must be %s %s, got %s %s" % (name, tuple(shape), dtype,
                                                             tuple(t.shape), t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _norm_topk(topk, levels):
    """an int (every level) or one value per level, as stored in the workspace record"""
    return int(topk) if isinstance(topk, int) else tuple(int(x) for x in topk)


def forward(q, k, v, topk, levels: int, flags: int = 0, workspace=None, stream=None):
    """Returns (out, lse, workspace); the workspace feeds `backward`.  topk: an
    int for every level, or one value per level (level 1 first).  The call
    records its shape, dtype, top-k, levels and flags on the returned
    workspace tensor; `backward` reuses and checks them."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    if not q.is_cuda:
        raise ValueError("q, k, v must be on a GPU (got %s)" % q.device)
    _check_tensors((("q", q), ("k", k), ("v", v)), q.shape, q.dtype, q.device)
    topk = _norm_topk(topk, levels)
    per_level = not isinstance(topk, int)
    nbytes = (llsa_workspace_bytes_lk if per_level else llsa_workspace_bytes)(
        B, H, N, d, 16, topk, levels, dt)
    if nbytes == 0:
        raise LlsaError(-2, "llsa_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif (not workspace.is_cuda or workspace.device != q.device or workspace.dtype != torch.uint8
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    (llsa_forward_lk if per_level else llsa_forward)(
        q, k, v, out, lse, B, H, N, d, 16, topk, levels, dt, flags, workspace,
        workspace.numel(), stream)
    workspace._llsa_forward = {"shape": (B, H, N, d), "dtype": q.dtype, "topk": topk,
                               "levels": int(levels), "flags": int(flags)}
    return out, lse, workspace


def forward_grid(q_raster, k_raster, v_raster, frames: int, height: int, width: int, topk: int,
                 levels: int, flags: int = 0, workspace=None, stream=None):
    """The forward on raster-order q, k, v [B, H, frames*height*width, d]:
    returns (q, k, v, out, lse, workspace) with q, k, v the grid-ordered
    copies (written by the pooling pass) that `backward` takes, and out, lse
    in grid order -- the results of grid_order and forward, bit for bit."""
    import torch
    if q_raster.dim() != 4:
        raise ValueError("q_raster must be [B, H, N, d]")
    B, H, N, d = q_raster.shape
    if N != frames * height * width:
        raise ValueError("N must equal frames*height*width")
    dt = _dtype_code(q_raster)
    if not q_raster.is_cuda:
        raise ValueError("q, k, v must be on a GPU (got %s)" % q_raster.device)
    _check_tensors((("q_raster", q_raster), ("k_raster", k_raster), ("v_raster", v_raster)),
                   q_raster.shape, q_raster.dtype, q_raster.device)
    if not isinstance(topk, int):
        raise ValueError("forward_grid takes one top-k for every level")
    nbytes = llsa_workspace_bytes(B, H, N, d, 16, topk, levels, dt)
    if nbytes == 0:
        raise LlsaError(-2, "llsa_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q_raster.device)
    elif (not workspace.is_cuda or workspace.device != q_raster.device
          or workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % q_raster.device)
    q, k, v, out = (torch.empty_like(q_raster) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q_raster.device)
    llsa_forward_grid(q_raster, k_raster, v_raster, q, k, v, out, lse, B, H, frames, height,
                      width, d, 16, topk, levels, dt, flags, workspace, workspace.numel(), stream)
    workspace._llsa_forward = {"shape": (B, H, N, d), "dtype": q.dtype, "topk": topk,
                               "levels": int(levels), "flags": int(flags)}
    return q, k, v, out, lse, workspace


def backward(q, k, v, out, lse, dout, topk=None, levels=None, workspace=None, flags=None,
             stream=None):
    """Returns (dq, dk, dv).  `workspace` must come from `forward` on the same
    q, k, v; topk, levels and flags default to the forward's and, if given,
    must equal them (a mismatch raises ValueError: the index lists in the
    workspace are laid out for the forward's values)."""
    import torch
    if workspace is None:
        raise ValueError("backward needs the workspace returned by forward")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    _check_tensors((("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)), q.shape,
                   q.dtype, q.device)
    _check_tensors((("lse", lse),), (B, H, N), torch.float32, q.device)
    rec = getattr(workspace, "_llsa_forward", None)
    given = {"topk": None if topk is None else _norm_topk(topk, levels), "levels": levels,
             "flags": flags}
    if rec is not None:
        if rec["shape"] != (B, H, N, d) or rec["dtype"] != q.dtype:
            raise ValueError("workspace holds a forward of shape %s %s, not %s %s"
                             % (rec["shape"], rec["dtype"], (B, H, N, d), q.dtype))
        for key, val in given.items():
            if val is not None and val != rec[key]:
                raise ValueError("%s=%r differs from the forward's %r" % (key, val, rec[key]))
        topk, levels, flags = rec["topk"], rec["levels"], rec["flags"]
    elif topk is None or levels is None:
        raise ValueError("topk and levels are needed for a workspace that forward() did not "
                         "return")
    flags = 0 if flags is None else flags
    if (not workspace.is_cuda or workspace.device != q.device or workspace.dtype != torch.uint8
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    (llsa_backward if isinstance(topk, int) else llsa_backward_lk)(
        q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, 16, topk, levels, dt, flags,
        workspace, workspace.numel(), stream)
    return dq, dk, dv


def zorder(x, side: int, inverse: bool = False, stream=None):
    """x [..., side*side, C] (contiguous) -> Z-ordered copy (or its inverse)."""
    import torch
    if not x.is_contiguous() or x.shape[-2] != side * side:
        raise ValueError("x must be contiguous with side*side tokens on dim -2")
    y = torch.empty_like(x)
    outer = x.numel() // (side * side * x.shape[-1])
    llsa_zorder(x, y, outer, side, x.shape[-1] * x.element_size(), int(inverse), stream)
    return y


def grid_order(x, frames: int, height: int, width: int, inverse: bool = False, stream=None):
    """x [..., frames*height*width, C] (contiguous, raster order) -> grid-ordered copy
    (or its inverse); frames == 1 for an image."""
    import torch
    n = frames * height * width
    if not x.is_contiguous() or x.shape[-2] != n:
        raise ValueError("x must be contiguous with frames*height*width tokens on dim -2")
    y = torch.empty_like(x)
    outer = x.numel() // (n * x.shape[-1])
    llsa_grid_order(x, y, outer, frames, height, width, x.shape[-1] * x.element_size(),
                    int(inverse), stream)
    return y
