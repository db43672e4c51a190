"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function declared in include/llsa.h, and
reject bad arguments before any HIP call.  The README's usage notes limit the
token count and top-k to powers of two; this library accepts any N that 16
divides (a partial last block at the coarser levels) and any top-k up to the
candidates a row of its level may have.
"""
import ctypes
import os
import subprocess

import pytest

import sparse_attention_diffusion_order_amd as L

pytestmark = pytest.mark.skipif(not os.path.exists(L.library_path()),
                                reason="libllsa.so not built")

BAD = 16  # a non-null address that validation must never dereference


def test_exports_every_declared_function():
    names = L.exported_names()
    assert {"llsa_forward", "llsa_backward", "llsa_zorder", "llsa_grid_order",
            "llsa_workspace_bytes",
            "llsa_workspace_layout", "llsa_strerror", "llsa_forward_part",
            "llsa_backward_part"} <= set(names)
    lib = L.load()
    for n in names:
        assert hasattr(lib, n), n
    syms = subprocess.run(["nm", "-D", "--defined-only", L.library_path()], capture_output=True,
                          text=True).stdout
    exported = {line.split()[-1] for line in syms.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n


def fwd(**kw):
    a = dict(q=BAD, k=BAD, v=BAD, out=BAD, lse=BAD, B=1, H=2, N=4096, d=64, block_size=16,
             topk=16, levels=1, dtype=L.BF16, flags=0, workspace=BAD, ws_bytes=1 << 40)
    a.update(kw)
    lib = L.load()
    return lib.llsa_forward(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"],
                            a["d"], a["block_size"], a["topk"], a["levels"], a["dtype"],
                            a["flags"], a["workspace"], a["ws_bytes"], None)


def bwd(**kw):
    a = dict(B=1, H=2, N=4096, d=64, block_size=16, topk=16, levels=1, dtype=L.BF16, flags=0,
             workspace=BAD, ws_bytes=1 << 40, dq=BAD)
    a.update(kw)
    lib = L.load()
    return lib.llsa_backward(BAD, BAD, BAD, BAD, BAD, BAD, a["dq"], BAD, BAD, a["B"], a["H"],
                             a["N"], a["d"], a["block_size"], a["topk"], a["levels"],
                             a["dtype"], a["flags"], a["workspace"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lse=None), -1),
    (dict(N=3000), -2), (dict(N=8), -2), (dict(topk=257), -2), (dict(topk=0), -2),
    (dict(N=48 * 80, levels=2, topk=16), -2),
    (dict(levels=0), -2), (dict(levels=4), -2), (dict(N=4096, levels=2, topk=32), -2),
    (dict(B=0), -2), (dict(H=-1), -2),
    (dict(d=96), -3), (dict(d=256), -3), (dict(block_size=32), -3), (dict(dtype=7), -3), (dict(flags=32), -3),
    (dict(N=65536, flags=8), -3),  # a complement of 4096 coarsest blocks: over 2048 entries
    (dict(flags=8 | 16), -3),      # the complement is not defined with causal
    (dict(flags=16, workspace=None), -4),  # causal: a known flag
    (dict(levels=7, N=1 << 30), -3), (dict(N=131072, topk=16), -3), (dict(topk=128, N=65536, levels=2), -3),
    (dict(B=1 << 16, H=1 << 4, N=4096), -3), (dict(N=1 << 24, levels=3, topk=16), -3),
    (dict(workspace=None), -4), (dict(ws_bytes=100), -4),
    # tensors move in 16-byte pieces, lse in 4-byte ones
    (dict(q=BAD + 8), -1), (dict(out=BAD + 4), -1), (dict(lse=BAD + 2), -1),
    (dict(lse=BAD + 4, workspace=None), -4), (dict(workspace=BAD + 8), -4),
])
def test_forward_validation(kw, code):
    assert fwd(**kw) == code
    if not {"q", "lse", "out"} & kw.keys():
        assert bwd(**{k: v for k, v in kw.items()}) == code


def test_backward_null_output():
    assert bwd(dq=None) == -1
    assert bwd(dq=BAD + 8) == -1


def test_zorder_validation():
    lib = L.load()
    assert lib.llsa_zorder(None, BAD, 1, 16, 128, 0, None) == -1
    assert lib.llsa_zorder(BAD, BAD, 1, 12, 128, 0, None) == -2
    assert lib.llsa_zorder(BAD, BAD, 1, 16, 6, 0, None) == -2
    assert lib.llsa_zorder(BAD, BAD, 0, 16, 128, 0, None) == -2


def test_grid_order_validation():
    lib = L.load()
    g = lib.llsa_grid_order
    assert g(None, BAD, 1, 1, 16, 16, 128, 0, None) == -1
    assert g(BAD, None, 1, 1, 16, 16, 128, 0, None) == -1
    assert g(BAD, BAD, 0, 1, 16, 16, 128, 0, None) == -2
    assert g(BAD, BAD, 1, 0, 16, 16, 128, 0, None) == -2
    assert g(BAD, BAD, 1, 1, 0, 16, 128, 0, None) == -2
    assert g(BAD, BAD, 1, 1, 16, 1 << 16, 128, 0, None) == -2
    assert g(BAD, BAD, 1, 1 << 10, 1 << 11, 1 << 10, 128, 0, None) == -2  # > 2^30 cells
    assert g(BAD, BAD, 1, 1, 16, 16, 6, 0, None) == -2


@pytest.mark.parametrize("N,K,Lv", [(48 * 80, 8, 2), (3 * 256, 3, 1), (15 * 256, 5, 2),
                                    (4 * 32 * 32, 12, 2), (3 * 4096, 3, 3)])
def test_shapes_beyond_powers_of_two_are_accepted(N, K, Lv):
    assert L.llsa_workspace_bytes(1, 2, N, 64, 16, K, Lv, L.BF16) > 0


def test_head_dimension_128_is_accepted():
    assert L.llsa_workspace_bytes(1, 2, 4096, 128, 16, 16, 2, L.BF16) > \
        L.llsa_workspace_bytes(1, 2, 4096, 64, 16, 16, 2, L.BF16) > 0


def test_per_level_top_k_validation():
    lib = L.load()
    arr = lambda *ks: (ctypes.c_int * len(ks))(*ks)
    wb = lambda ks, N=4096, Lv=2: lib.llsa_workspace_bytes_lk(1, 2, N, 64, 16, ks, Lv, L.BF16)
    lay = L.WsLayout()
    assert lib.llsa_workspace_layout_lk(1, 2, 4096, 64, 16, None, 2, L.BF16,
                                        ctypes.byref(lay)) == -1
    assert wb(arr(8, 4)) > 0
    assert wb(arr(16, 16)) == L.llsa_workspace_bytes(1, 2, 4096, 64, 16, 16, 2, L.BF16)
    assert wb(arr(8, 17)) == 0          # coarsest: 16 blocks
    assert wb(arr(65, 4)) == 0          # level 1: at most 16 * 4 = 64 candidates
    assert wb(arr(0, 4)) == 0
    assert wb(arr(2, 3, 1), N=4096, Lv=3) > 0
    assert wb(arr(2, 17, 1), N=4096, Lv=3) == 0  # 16 * 1 level-2 candidates
    args = [BAD] * 5 + [1, 2, 4096, 64, 16]
    assert lib.llsa_forward_lk(*args, None, 2, L.BF16, 0, BAD, 1 << 40, None) == -1
    assert lib.llsa_forward_lk(*args, arr(8, 17), 2, L.BF16, 0, BAD, 1 << 40, None) == -2
    assert lib.llsa_forward_lk(*args, arr(128, 16), 2, L.BF16, 0, BAD, 1 << 40, None) == -3
    assert lib.llsa_forward_lk(*args, arr(8, 4), 2, L.BF16, 0, BAD, 100, None) == -4
    bargs = [BAD] * 9 + [1, 2, 4096, 64, 16]
    assert lib.llsa_backward_lk(*bargs, arr(8, 17), 2, L.BF16, 0, BAD, 1 << 40, None) == -2
    # each level's lists take that level's top-k
    lk = L.llsa_workspace_layout_lk(1, 2, 4096, 64, 16, [8, 4], 2, L.BF16)
    assert lk["idx"][1] - lk["idx"][0] >= 2 * 256 * 8 * 4
    assert lk["col"][1] - lk["col"][0] >= 2 * 256 * 8 * 4


def test_strerror():
    for c in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(L.llsa_strerror(c), str) and L.llsa_strerror(c)


def test_workspace_is_log_linear_not_quadratic():
    # the backward keeps sparse lists only: workspace grows linearly with N
    small = L.llsa_workspace_bytes(1, 1, 65536, 64, 16, 16, 2, L.BF16)
    big = L.llsa_workspace_bytes(1, 1, 262144, 64, 16, 16, 2, L.BF16)
    assert 3.5 < big / small < 4.5
    assert L.llsa_workspace_bytes(1, 1, 3000, 64, 16, 16, 1, L.BF16) == 0


@pytest.mark.parametrize("B,H,N,K,Lv", [(1, 1, 1024, 8, 1), (1, 6, 65536, 16, 2),
                                        (1, 6, 262144, 16, 3)])
def test_layout_consistent(B, H, N, K, Lv):
    lay = L.llsa_workspace_layout(B, H, N, 64, 16, K, Lv, L.BF16)
    assert lay["total"] == L.llsa_workspace_bytes(B, H, N, 64, 16, K, Lv, L.BF16)
    G = B * H
    spans = []
    for l in range(1, Lv + 1):
        n = N // 16 ** l
        for name, size in (("qbar", G * n * 64 * 4), ("kbar", G * n * 64 * 4),
                           ("vbar", G * n * 64 * 4), ("idx", G * n * K * 4),
                           ("rowptr", G * (n + 1) * 4), ("col", G * n * K * 4)):
            spans.append((lay[name][l - 1], size))
    spans.append((lay["delta"], G * N * 4))
    spans.sort()
    for (a, sa), (b, _) in zip(spans, spans[1:]):
        assert a % 256 == 0 and a + sa <= b  # aligned and disjoint
    assert spans[-1][0] + spans[-1][1] <= lay["total"]


def test_binding_refuses_host_tensors_and_mismatched_backward():
    """The Python helpers check device, shape, dtype and contiguity before any
    library call (a host tensor's address must never reach a kernel), and the
    backward refuses top-k, levels or flags other than the forward's."""
    import torch
    q = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.forward(q, q, q, 4, 1)
    with pytest.raises(ValueError):
        L.llsa_zorder(q, q, 2, 16, 128)
    ws = torch.zeros(16, dtype=torch.uint8)
    ws._llsa_forward = {"shape": (1, 2, 256, 64), "dtype": torch.bfloat16, "topk": 4,
                        "levels": 1, "flags": 0}
    lse = torch.zeros(1, 2, 256)
    with pytest.raises(ValueError):  # host tensors
        L.backward(q, q, q, q, lse, q, workspace=ws)
    with pytest.raises(ValueError):  # no workspace
        L.backward(q, q, q, q, lse, q, 4, 1)


def test_noalloc_forward_refuses_oversized_shapes_before_any_launch():
    """The allocation-free forward checks its arguments, then whether the
    shape's forward state fits the static scratch, before any HIP call."""
    lib = L.load()
    args = (BAD, BAD, BAD, BAD, BAD)
    # 512^2 tokens, 6 heads, 3 levels: about 120 MB of forward state
    assert lib.llsa_forward_noalloc(*args, 1, 6, 262144, 64, 16, 16, 3, L.BF16, 0, None) == -6
    assert lib.llsa_forward_noalloc(None, BAD, BAD, BAD, BAD, 1, 6, 4096, 64, 16, 16, 1,
                                    L.BF16, 0, None) == -1
    assert lib.llsa_forward_noalloc(*args, 1, 6, 4008, 64, 16, 16, 1, L.BF16, 0, None) == -2
    assert lib.llsa_forward_noalloc(*args, 1, 6, 4096, 96, 16, 16, 1, L.BF16, 0, None) == -3
    assert "scratch" in L.llsa_strerror(-6)


@pytest.mark.parametrize("N,K,Lv,ok", [
    (336, (4, 2), 2, True),     # 21 level-1 blocks, level-2 blocks of 16 and 5
    (336, (21, 2), 2, True),    # a level-1 row may have 16 + 5 = 21 candidates
    (336, (22, 2), 2, False),
    (336, (4, 3), 2, False),    # only 2 level-2 blocks
    (336, (5, 1), 2, True),     # a row under the partial block has 5 candidates
    (336, (6, 1), 2, False),
    (10000, (16, 16), 2, True), # 100 x 100: 625 level-1 and 40 level-2 blocks
    (4800, (8, 4, 2), 3, True), # 300 / 19 / 2 blocks
    (4808, (4, 2), 2, False),   # not a multiple of 16
])
def test_token_counts_that_16_to_the_levels_does_not_divide(N, K, Lv, ok):
    nb = L.llsa_workspace_bytes_lk(1, 2, N, 64, 16, list(K), Lv, L.BF16)
    assert (nb > 0) == ok
    lib = L.load()
    arr = (ctypes.c_int * Lv)(*K)
    rc = lib.llsa_forward_lk(BAD, BAD, BAD, BAD, BAD, 1, 2, N, 64, 16, arr, Lv, L.BF16, 0, BAD, 0,
                             None)
    assert rc == (-4 if ok else -2)  # a valid shape then fails on the missing workspace


def _fwd_grid(**kw):
    a = dict(ptrs=[BAD] * 8, B=1, H=2, frames=1, height=64, width=64, d=64, block_size=16,
             topk=16, levels=2, dtype=L.BF16, flags=0, workspace=BAD, ws_bytes=1 << 40)
    a.update(kw)
    return L.load().llsa_forward_grid(*a["ptrs"], a["B"], a["H"], a["frames"], a["height"],
                                      a["width"], a["d"], a["block_size"], a["topk"],
                                      a["levels"], a["dtype"], a["flags"], a["workspace"],
                                      a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ptrs=[None] + [BAD] * 7), -1), (dict(ptrs=[BAD] * 5 + [None] + [BAD] * 2), -1),
    (dict(ptrs=[BAD] * 7 + [None]), -1),
    (dict(height=0), -2), (dict(width=1 << 16), -2), (dict(frames=-1), -2),
    (dict(height=3, width=5), -2),            # N = 15: not a multiple of 16
    (dict(height=16, width=21, topk=2), -4),  # N = 336: valid, no workspace given
    (dict(height=16, width=21), -2),          # top-16 of two level-2 blocks
    (dict(frames=4, height=32, width=32), -4),
    (dict(d=96), -3), (dict(flags=32), -3), (dict(topk=0), -2),
    (dict(workspace=None), -4), (dict(ws_bytes=100), -4),
])
def test_forward_grid_validation(kw, code):
    if code == -4 and "workspace" not in kw and "ws_bytes" not in kw:
        kw = dict(kw, workspace=None)
    assert _fwd_grid(**kw) == code
