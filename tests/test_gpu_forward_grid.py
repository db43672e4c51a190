"""llsa_forward_grid (the grid order folded into the pooling pass) against
llsa_grid_order followed by llsa_forward, through the C ABI: the grid-ordered
copies of q, k, v, out, lse and the workspace's pyramid and index lists are
identical bit for bit, and so are the gradients of a backward from either.

Grids: a square power-of-two image (one tile), rectangles whose tiles hold
16 or more cells (one raster cell per token at a block-base offset) and
fewer (S = 2 and S = 1: the per-token mapping), video, fp32, d = 128, a
token count that 16^levels does not divide, and the causal flag.
"""
import numpy as np
import pytest

import synth
from llsa_check import to_device

pytestmark = pytest.mark.gpu

W = synth.Workload


def _w(name, dtype, L, K, side, height=0, frames=1, H=2, d=64):
    return W(name, 1, H, side, d, dtype, L, K, 2.0, 0, 16, frames, height)


_CASES = [
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), 0),
    (synth.WORKLOADS["grid256_bf16_l2_k16"], 0),
    (_w("rect48x80_bf16_l2_k4", "bf16", 2, 4, 80, height=48), 0),      # S = 16
    (_w("rect12x20_bf16_l1_k3", "bf16", 1, 3, 20, height=12), 0),      # S = 4
    (_w("rect18x40_bf16_l1_k4", "bf16", 1, 4, 40, height=18), 0),      # S = 2: per token
    (_w("rect16x21_bf16_l2_k4x2", "bf16", 2, 2, 21, height=16), 0),    # S = 1, N = 336
    (_w("video4x32x32_bf16_l2_k4", "bf16", 2, 4, 32, frames=4), 0),    # S = 4 (cubes)
    (_w("video2x16x24_bf16_l1_k4", "bf16", 1, 4, 24, height=16, frames=2), 0),  # S = 2
    (_w("grid32_f32_l2_k2", "f32", 2, 2, 32), 0),
    (_w("rect48x80_f32_l1_k4", "f32", 1, 4, 80, height=48, H=1), 0),
    (_w("grid64_bf16_l2_k4_d128", "bf16", 2, 4, 64, d=128), 0),
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), 16),                   # causal
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), 4 | 2),                # size bias, coarse
]


@pytest.mark.parametrize("w,flags", _CASES, ids=["%s_f%d" % (w.name, f) for w, f in _CASES])
def test_forward_grid_matches_grid_order_then_forward(w, flags):
    import torch
    import sparse_attention_diffusion_order_amd as lib
    inp = synth.make_inputs(w)
    q_r, k_r, v_r = (to_device(inp[n], w.dtype) for n in ("q", "k", "v"))
    q0, k0, v0 = (lib.grid_order(x, w.frames, w.rows, w.side) for x in (q_r, k_r, v_r))
    out0, lse0, ws0 = lib.forward(q0, k0, v0, w.topk, w.levels, flags)
    q1, k1, v1, out1, lse1, ws1 = lib.forward_grid(q_r, k_r, v_r, w.frames, w.rows, w.side,
                                                   w.topk, w.levels, flags)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else (lambda t: t.view(torch.int32))
    for a, b, name in ((q1, q0, "q"), (k1, k0, "k"), (v1, v0, "v"), (out1, out0, "out")):
        assert torch.equal(bits(a), bits(b)), name
    assert torch.equal(lse1.view(torch.int32), lse0.view(torch.int32))
    # the forward's state: pyramid, bf16 copies and index lists (every byte
    # the forward writes; the backward's parts are not written yet)
    lay = lib.llsa_workspace_layout(w.B, w.H, w.N, w.d, 16, w.topk, w.levels,
                                    lib.BF16 if w.dtype == "bf16" else lib.F32)
    for l in range(w.levels):
        n = -(-w.N // 16 ** (l + 1))
        for name, nbytes in (("qbar", n * w.d * 4), ("kbar", n * w.d * 4), ("vbar", n * w.d * 4),
                             ("idx", n * w.topk * 4)):
            off, size = lay[name][l], w.G * nbytes
            assert torch.equal(ws1[off:off + size], ws0[off:off + size]), (name, l + 1)
    if w.N <= 4096:
        do = to_device(inp["do"], w.dtype)
        g0 = lib.backward(q0, k0, v0, out0, lse0, do, w.topk, w.levels, ws0, flags)
        g1 = lib.backward(q1, k1, v1, out1, lse1, do, w.topk, w.levels, ws1, flags)
        torch.cuda.synchronize()
        for a, b in zip(g1, g0):
            assert torch.equal(bits(a), bits(b))
