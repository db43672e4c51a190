"""Python side of the LLSA CPU oracle (plain fp64 C, see llsa_oracle.h).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py; the product path never imports it.  It shares no
code with the HIP library; it only marshals numpy arrays into the C routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "llsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
NO_ENRICH = 1
ENRICH_COARSE = 2
SIZE_BIAS = 4
ENRICH_COMPLEMENT = 8
CAUSAL = 16

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.orc_morton.argtypes = [I, I, I]
        lib.orc_morton.restype = I
        lib.orc_zorder.argtypes = [P, P, I, I, I, ctypes.c_int]
        lib.orc_grid_index.argtypes = [I] * 6
        lib.orc_grid_index.restype = I
        lib.orc_grid_order.argtypes = [P, P, I, I, I, I, I, ctypes.c_int]
        lib.orc_pool.argtypes = [P, I, I, I, I, ctypes.c_int, P]
        lib.orc_select_level.argtypes = [P, P, P, I, I, I, I, I, I, D, ctypes.c_int, P, P]
        lib.orc_select.argtypes = [P, P, I, I, I, I, ctypes.c_int, P, D, ctypes.c_int, P, P]
        lib.orc_forward.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_int, P, D,
                                    ctypes.c_uint, P, I, P, P]
        lib.orc_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, ctypes.c_int,
                                     P, D, ctypes.c_uint, P, I, P, I, P, P, P]
        lib.orc_transpose.argtypes = [P, I, I, I, P, P]
        for f in ("orc_zorder", "orc_grid_order", "orc_pool", "orc_select_level", "orc_select",
                  "orc_forward", "orc_backward", "orc_transpose"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def level_sizes(N: int, bs: int, L: int):
    """blocks per level: ceil(N / bs^l) (the last block of a level may be partial)"""
    return [-(-N // bs ** l) for l in range(1, L + 1)]


def min_candidates(N: int, bs: int, L: int, K):
    """The fewest candidates any row of each level has (level 1 first): every
    block at the coarsest level; below it the existing children of the
    parent's picks, at worst bs (K_{l+1} - 1) full parents and the partial last
    one."""
    ks = level_topk(K, L)
    n = level_sizes(N, bs, L)
    out = []
    for l in range(1, L + 1):
        if l == L:
            out.append(n[l - 1])
        else:
            last = n[l - 1] - bs * (n[l] - 1)  # children of the last parent block
            out.append(bs * (ks[l] - 1) + last)
    return out


def check_topk(N: int, bs: int, L: int, K):
    """Raise ValueError unless every row has at least as many candidates as picks."""
    for l, (k, m) in enumerate(zip(level_topk(K, L), min_candidates(N, bs, L, K)), 1):
        if k > m:
            raise ValueError("level %d: top-k %d exceeds the %d candidates a row may have"
                             % (l, k, m))


def _flat_levels(levels):
    """[G, n_l, w] per level -> one buffer, level-major (the C pyramid layout)."""
    return np.ascontiguousarray(np.concatenate([np.ravel(_f64(x)) if x.dtype != np.int32
                                                else np.ravel(x) for x in levels]))


def _split_levels(buf, G, sizes, w, squeeze=False):
    out, off = [], 0
    for n in sizes:
        seg = buf[off:off + G * n * w]
        out.append(seg.reshape(G, n) if squeeze else seg.reshape(G, n, w))
        off += G * n * w
    return out


def morton(side: int, y: int, x: int) -> int:
    return int(_load().orc_morton(side, y, x))


def zorder(x, side: int, inverse: bool = False):
    """x [outer, side*side, inner] -> Z-ordered copy (or its inverse)."""
    x = _f64(x)
    outer, n, inner = x.shape
    assert n == side * side
    y = np.empty_like(x)
    _load().orc_zorder(_p(x), _p(y), outer, side, inner, int(inverse))
    return y


def grid_index(frames: int, height: int, width: int, t: int, y: int, x: int) -> int:
    return int(_load().orc_grid_index(frames, height, width, t, y, x))


def grid_order(x, frames: int, height: int, width: int, inverse: bool = False):
    """x [outer, frames*height*width, inner] (raster order) -> grid order (or back)."""
    x = _f64(x)
    outer, n, inner = x.shape
    assert n == frames * height * width
    y = np.empty_like(x)
    _load().orc_grid_order(_p(x), _p(y), outer, frames, height, width, inner, int(inverse))
    return y


def pool(x, bs: int, L: int):
    """x [G, N, d] -> [level 1, ..., level L], each [G, N/bs^l, d]."""
    x = _f64(x)
    G, N, d = x.shape
    sizes = level_sizes(N, bs, L)
    buf = np.zeros(G * d * sum(sizes))
    _load().orc_pool(_p(x), G, N, d, bs, L, _p(buf))
    return _split_levels(buf, G, sizes, d)


def level_topk(K, L: int):
    """K as an int (every level) or a sequence of L values (level 1 first)."""
    ks = [int(K)] * L if np.isscalar(K) else [int(x) for x in K]
    assert len(ks) == L
    return ks


def _ks(idx):
    """per-level K of an index pyramid, as the C array the oracle takes"""
    return np.ascontiguousarray([x.shape[2] for x in idx], dtype=np.int64)


def select_level(qbar, kbar, parent, K: int, bs: int, scale: float, causal: bool = False):
    """One level of Top-K; returns (idx [G, n, K] int32, gap [G, n]).  The
    parent rows may hold another count of picks than K.  causal: each row
    keeps itself and its best K-1 earlier candidates (-1 in unused slots)."""
    qbar, kbar = _f64(qbar), _f64(kbar)
    G, n, d = qbar.shape
    par = None if parent is None else _i32(parent)
    Kp = 0 if par is None else par.shape[2]
    if par is not None:
        assert par.shape[:2] == (G, -(-n // bs))
    idx = np.zeros((G, n, K), np.int32)
    gap = np.zeros((G, n))
    _load().orc_select_level(_p(qbar), _p(kbar), _p(par), G, n, d, bs, K, Kp, scale,
                             int(causal), _p(idx), _p(gap))
    return idx, gap


def select(qpyr, kpyr, K, bs: int, scale: float, N=None, causal: bool = False):
    """All levels; K an int or one value per level (level 1 first); N: the
    token count (default: level 1's blocks times bs).  Returns (idx list per
    level 1..L, gap list per level)."""
    G, n1, d = qpyr[0].shape
    L = len(qpyr)
    N = n1 * bs if N is None else N
    ks = level_topk(K, L)
    if not causal:  # causal rows may keep fewer picks (-1 in the slots left)
        check_topk(N, bs, L, ks)
    sizes = level_sizes(N, bs, L)
    idx = np.zeros(G * sum(n * k for n, k in zip(sizes, ks)), np.int32)
    gap = np.zeros(G * sum(sizes))
    ka = np.ascontiguousarray(ks, dtype=np.int64)
    _load().orc_select(_p(_flat_levels(qpyr)), _p(_flat_levels(kpyr)), G, N, d, bs, L, _p(ka),
                       scale, int(causal), _p(idx), _p(gap))
    out, off = [], 0
    for n, k in zip(sizes, ks):
        out.append(idx[off:off + G * n * k].reshape(G, n, k))
        off += G * n * k
    return out, _split_levels(gap, G, sizes, 1, squeeze=True)


def forward(q, k, v, kpyr, vpyr, idx, bs: int, scale: float, flags: int = 0,
            qblocks=None, out=None, lse=None):
    """Sparse attention forward; returns (out [G, N, d], lse [G, N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    G, N, d = q.shape
    L, K = len(idx), _ks(idx)
    out = np.zeros((G, N, d)) if out is None else out
    lse = np.zeros((G, N)) if lse is None else lse
    qb = None if qblocks is None else np.ascontiguousarray(qblocks, dtype=np.int64)
    _load().orc_forward(_p(q), _p(k), _p(v), _p(_flat_levels(kpyr)), _p(_flat_levels(vpyr)),
                        _p(_flat_levels([_i32(x) for x in idx])), G, N, d, bs, L, _p(K),
                        scale, flags, _p(qb), 0 if qb is None else len(qb), _p(out), _p(lse))
    return out, lse


def backward(q, k, v, kpyr, vpyr, idx, o, lse, dout, bs: int, scale: float,
             flags: int = 0, qblocks=None, kblocks=None):
    """Backward; returns (dq, dk, dv), each [G, N, d] (only requested rows set)."""
    q, k, v, o, lse, dout = (_f64(a) for a in (q, k, v, o, lse, dout))
    G, N, d = q.shape
    L, K = len(idx), _ks(idx)
    dq, dk, dv = (np.zeros((G, N, d)) for _ in range(3))
    qb = None if qblocks is None else np.ascontiguousarray(qblocks, dtype=np.int64)
    kb = None if kblocks is None else np.ascontiguousarray(kblocks, dtype=np.int64)
    _load().orc_backward(_p(q), _p(k), _p(v), _p(_flat_levels(kpyr)), _p(_flat_levels(vpyr)),
                         _p(_flat_levels([_i32(x) for x in idx])), _p(o), _p(lse), _p(dout),
                         G, N, d, bs, L, _p(K), scale, flags, _p(qb), 0 if qb is None else len(qb),
                         _p(kb), 0 if kb is None else len(kb), _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


def transpose(idx):
    """idx [G, n, K] -> (rowptr [G, n+1], col [G, n*K]) with ascending rows."""
    idx = _i32(idx)
    G, n, K = idx.shape
    rowptr = np.zeros((G, n + 1), np.int32)
    col = np.zeros((G, n * K), np.int32)
    _load().orc_transpose(_p(idx), G, n, K, _p(rowptr), _p(col))
    return rowptr, col


def run(q, k, v, bs: int, L: int, K, flags: int = 0, dout=None, scale=None,
        idx=None, qblocks=None):
    """Whole path on Z-ordered [G, N, d] inputs: pyramid, selection (unless
    `idx` is given; K an int or one value per level), forward and, with `dout`,
    backward.  Returns a dict."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape[1], q.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qp, kp, vp = pool(q, bs, L), pool(k, bs, L), pool(v, bs, L)
    gap = None
    if idx is None:
        idx, gap = select(qp, kp, K, bs, scale, N=N, causal=bool(flags & CAUSAL))
    res = {"qpyr": qp, "kpyr": kp, "vpyr": vp, "idx": idx, "gap": gap, "scale": scale}
    if dout is None:
        res["out"], res["lse"] = forward(q, k, v, kp, vp, idx, bs, scale, flags, qblocks)
        return res
    res["out"], res["lse"] = forward(q, k, v, kp, vp, idx, bs, scale, flags)
    res["dq"], res["dk"], res["dv"] = backward(q, k, v, kp, vp, idx, res["out"], res["lse"],
                                               dout, bs, scale, flags)
    return res
