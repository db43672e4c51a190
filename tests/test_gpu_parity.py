"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Comparison rules are in llsa_check.py.

Where the bf16 path legitimately picks a different block (oracle gap < 1e-3),
the oracle's forward/backward is re-run on the GPU's index lists, so values
are compared for the same key/value sets; the index lists themselves are
checked separately against the oracle's selection.
"""
import numpy as np
import pytest

import oracle
import synth
from llsa_check import (BS, TOL, assert_close, check_selection, check_transpose, full_check,
                        gpu_run, grad_tol, oracle_inputs, oracle_values, to_device, ws_array)

pytestmark = pytest.mark.gpu

W = synth.Workload


def small(name, B, H, side, dtype, L, K, sigma=2.0, seed=0):
    return W(name, B, H, side, 64, dtype, L, K, sigma, seed)


SMALL = [
    synth.WORKLOADS["grid32_f32_l1_k8"],
    small("grid32_f32_l2_k2", 1, 2, 32, "f32", 2, 2),
    small("grid16_bf16_l1_k4", 1, 3, 16, "bf16", 1, 4),
    small("grid32_bf16_l2_k2", 2, 1, 32, "bf16", 2, 2),
    small("grid64_bf16_l2_k4", 1, 2, 64, "bf16", 2, 4),
    small("grid64_bf16_l3_k1", 1, 2, 64, "bf16", 3, 1),
    small("grid64_bf16_l1_k32", 1, 1, 64, "bf16", 1, 32),
    synth.WORKLOADS["grid64_bf16_l1_k16"],
    # two levels with top-16 at both: at 64^2 the coarsest level has exactly
    # 16 blocks, so every coarsest row picks all of them
    small("grid64_bf16_l2_k16", 2, 3, 64, "bf16", 2, 16),
    W("rect64x128_bf16_l2_k16", 1, 2, 128, 64, "bf16", 2, 16, 2.0, 0, 16, 1, 64),
]


_full_check = full_check


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_workloads(w):
    _full_check(w)


@pytest.mark.parametrize("w", [
    # topk = 64 at a 1024-block coarsest level: the selection's score tile
    # needs more than 64 KiB of LDS; the attention uses the one-block kernels
    small("grid128_bf16_l1_k64", 1, 1, 128, "bf16", 1, 64),
    # a 4096-block coarsest level: the dense selection with few rows per
    # workgroup
    small("grid256_bf16_l1_k16", 1, 1, 256, "bf16", 1, 16),
], ids=lambda w: w.name)
def test_large_candidate_lists(w):
    _full_check(w)


@pytest.mark.parametrize("w", [SMALL[0], SMALL[4]], ids=lambda w: w.name)
def test_no_enrichment(w):
    _full_check(w, flags=oracle.NO_ENRICH)


_COARSE, _SIZE = oracle.ENRICH_COARSE, oracle.SIZE_BIAS
_VARIANT_CASES = [
    (SMALL[0], _SIZE),  # fp32, one level
    (SMALL[2], _SIZE),  # bf16, one level (four-block kernel)
    (SMALL[1], _COARSE), (SMALL[1], _SIZE), (SMALL[1], _COARSE | _SIZE),
    (SMALL[4], _COARSE), (SMALL[4], _SIZE), (SMALL[4], _COARSE | _SIZE),
    (SMALL[5], _COARSE | _SIZE),  # three levels, topk 1
    (SMALL[6], _COARSE),  # one level: coarse enrichment adds nothing
    # topk 32 over two levels: the one-block bf16 kernels
    (small("grid128_bf16_l2_k32", 1, 1, 128, "bf16", 2, 32), _COARSE | _SIZE),
    (small("grid128_bf16_l2_k32", 1, 1, 128, "bf16", 2, 32), _SIZE),
]


@pytest.mark.parametrize("w,flags", _VARIANT_CASES,
                         ids=["%s_f%d" % (w.name, f) for w, f in _VARIANT_CASES])
def test_enrichment_variants(w, flags):
    _full_check(w, flags=flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zorder_gather_bit_exact(dtype):
    import torch
    import sparse_attention_diffusion_order_amd as lib
    from llsa_check import to_device
    w = small("z", 2, 3, 64, dtype, 1, 1)
    inp = synth.make_inputs(w, want_grad=False)
    x = to_device(inp["q"], dtype)
    z = lib.zorder(x, w.side)
    back = lib.zorder(z, w.side, inverse=True)
    torch.cuda.synchronize()
    want = oracle.zorder(inp["q64"].reshape(w.G, w.N, w.d), w.side)
    got = z.float().cpu().numpy().astype(np.float64).reshape(w.G, w.N, w.d)
    np.testing.assert_array_equal(got, want)
    assert torch.equal(back.view(torch.int16) if dtype == "bf16" else back,
                       x.view(torch.int16) if dtype == "bf16" else x)
    # odd row width (12 bytes) exercises the 4-byte path
    y = torch.arange(4 * 16 * 3, dtype=torch.float32, device="cuda").reshape(4, 16, 3)
    yz = lib.zorder(y, 4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(yz.cpu().numpy(),
                                  oracle.zorder(y.cpu().numpy(), 4).astype(np.float32))


@pytest.mark.parametrize("T,Hh,Ww", [(1, 48, 80), (1, 16, 64), (1, 12, 20), (1, 3, 5),
                                     (4, 32, 32), (3, 8, 24), (2, 16, 16), (8, 4, 4)])
@pytest.mark.parametrize("dtype,width", [("f32", 64), ("bf16", 64), ("f32", 3), ("f32", 2),
                                         ("bf16", 2)])  # rows of 256, 128, 12, 8, 4 bytes
def test_grid_order_bit_exact(T, Hh, Ww, dtype, width):
    import torch
    import sparse_attention_diffusion_order_amd as lib
    n = T * Hh * Ww
    rng = np.random.default_rng(n + width)
    for dt in ((torch.float32,) if dtype == "f32" else (torch.bfloat16,)):
        x = torch.from_numpy(rng.standard_normal((2, n, width))).to(dt).cuda()
        z = lib.grid_order(x, T, Hh, Ww)
        back = lib.grid_order(z, T, Hh, Ww, inverse=True)
        torch.cuda.synchronize()
        x64 = x.float().cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(z.float().cpu().numpy(), oracle.grid_order(x64, T, Hh, Ww))
        assert torch.equal(back.view(torch.int16) if dt == torch.bfloat16 else back,
                           x.view(torch.int16) if dt == torch.bfloat16 else x)


def _grid(name, dtype, L, K, side, height=0, frames=1, B=1, H=2, sigma=2.0, d=64):
    return W(name, B, H, side, d, dtype, L, K, sigma, 0, 16, frames, height)


# shapes the README's power-of-two limits exclude: rectangles, odd top-k,
# block counts that are not multiples of 4 or 16, and video in octree order
_BEYOND = [
    _grid("rect48x80_bf16_l2_k8", "bf16", 2, 8, 80, height=48),     # N = 3840, 15 coarse blocks
    _grid("rect12x20_bf16_l1_k4", "bf16", 1, 4, 20, height=12),     # 15 blocks: one-block kernels
    _grid("rect12x20_f32_l1_k3", "f32", 1, 3, 20, height=12),
    _grid("grid64_bf16_l1_k12", "bf16", 1, 12, 64),                 # topk 12
    _grid("grid32_f32_l2_k3", "f32", 2, 3, 32),                     # topk 3 of 4 coarse blocks
    _grid("rect96x128_bf16_l3_k2", "bf16", 3, 2, 128, height=96, H=1),  # N = 12288, 3 coarse
    _grid("video4x32x32_bf16_l2_k8", "bf16", 2, 8, 32, frames=4),   # octree, N = 4096
    _grid("video2x16x16_f32_l1_k4", "f32", 1, 4, 16, frames=2, H=1),
    _grid("video3x16x16_bf16_l2_k2", "bf16", 2, 2, 16, frames=3),   # 3 coarse blocks
    # odd top-k on the bf16 kernels: the four-block forward (64 blocks),
    # the one-block forward (15 blocks), two levels, d = 128
    _grid("grid64_bf16_l1_k3", "bf16", 1, 3, 64),
    _grid("grid64_bf16_l2_k5", "bf16", 2, 5, 64),
    _grid("rect12x20_bf16_l1_k3", "bf16", 1, 3, 20, height=12),
    _grid("grid128_bf16_l2_k7", "bf16", 2, 7, 128, H=1),
    _grid("grid64_bf16_l2_k5_d128", "bf16", 2, 5, 64, d=128),
    _grid("grid64_bf16_l1_k33", "bf16", 1, 33, 64, H=1),            # odd and > 32
]


@pytest.mark.parametrize("w", _BEYOND, ids=lambda w: w.name)
def test_shapes_beyond_powers_of_two(w):
    _full_check(w)


# a top-k per level (level 1 first), through the _lk entry points
_PER_LEVEL = [
    (_grid("grid64_bf16_l2_k8x4", "bf16", 2, (8, 4), 64), 0),           # four-block kernels
    (_grid("grid128_bf16_l2_k32x8", "bf16", 2, (32, 8), 128), 0),       # one-block kernels
    (_grid("grid32_f32_l2_k4x2", "f32", 2, (4, 2), 32), 0),
    (_grid("grid64_bf16_l3_k2x3x1", "bf16", 3, (2, 3, 1), 64), 0),
    (_grid("grid128_bf16_l2_k32x8", "bf16", 2, (32, 8), 128),
     oracle.ENRICH_COARSE | oracle.SIZE_BIAS),
    (_grid("grid64_bf16_l2_k8x4", "bf16", 2, (8, 4), 64), oracle.SIZE_BIAS),
    (_grid("grid32_f32_l2_k4x2", "f32", 2, (4, 2), 32), oracle.SIZE_BIAS),
    (_grid("grid64_bf16_l2_k2x16", "bf16", 2, (2, 16), 64), 0),         # fewer fine picks
    # every coarsest block picked: the fused two-level selection with 1024
    # candidates per fine row (its largest LDS tile)
    (_grid("grid128_bf16_l2_k16x64", "bf16", 2, (16, 64), 128, H=1), 0),
]


@pytest.mark.parametrize("w,flags", _PER_LEVEL,
                         ids=["%s_f%d" % (w.name, f) for w, f in _PER_LEVEL])
def test_top_k_per_level(w, flags):
    _full_check(w, flags=flags)


# token counts that 16^levels does not divide (a multiple of 16): partial
# last blocks at the coarser levels, whose pooled tokens average fewer tokens,
# and rows whose parent is such a block, which have fewer candidates
_PADDED = [
    (_grid("grid16x21_bf16_l2_k4x2", "bf16", 2, (4, 2), 21, height=16), 0),      # N = 336
    (_grid("grid16x21_f32_l2_k4x2", "f32", 2, (4, 2), 21, height=16), 0),
    (_grid("grid16x21_bf16_l2_k5x1", "bf16", 2, (5, 1), 21, height=16), 0),      # 5 candidates
    (_grid("grid16x21_bf16_l2_k21x2", "bf16", 2, (21, 2), 21, height=16, H=1), 0),  # every block
    (_grid("grid16x21_bf16_l2_k4x2", "bf16", 2, (4, 2), 21, height=16), oracle.SIZE_BIAS),
    (_grid("grid16x21_bf16_l2_k4x2", "bf16", 2, (4, 2), 21, height=16), oracle.ENRICH_COARSE),
    (_grid("rect100x100_bf16_l2_k16", "bf16", 2, 16, 100, height=100), 0),       # N = 10000
    (_grid("rect60x80_bf16_l3_k8x4x2", "bf16", 3, (8, 4, 2), 80, height=60), 0),  # N = 4800
    (_grid("rect60x80_f32_l3_k8x4x2", "f32", 3, (8, 4, 2), 80, height=60, H=1), 0),
    (_grid("rect100x100_bf16_l2_k16_d128", "bf16", 2, 16, 100, height=100, d=128), 0),
    (_grid("rect100x100_bf16_l2_k16", "bf16", 2, 16, 100, height=100), oracle.NO_ENRICH),
]


@pytest.mark.parametrize("w,flags", _PADDED, ids=["%s_f%d" % (w.name, f) for w, f in _PADDED])
def test_token_counts_beyond_16_to_the_levels(w, flags):
    _full_check(w, flags=flags)


# the complement variant: the pooled tokens of the candidates a level did
# not pick (oracle.ENRICH_COMPLEMENT), alone and with the other flags
_CMP = oracle.ENRICH_COMPLEMENT
_COMPLEMENT = [
    (SMALL[0], _CMP), (SMALL[0], _CMP | _SIZE),                        # fp32, one level
    (SMALL[1], _CMP), (SMALL[1], _CMP | _SIZE | _COARSE),              # fp32, two levels
    (SMALL[4], _CMP), (SMALL[4], _CMP | _SIZE), (SMALL[4], _CMP | _COARSE),
    (SMALL[5], _CMP),                                                  # three levels, topk 1
    (synth.WORKLOADS["grid64_bf16_l1_k16"], _CMP),                     # 240 entries per block
    (_grid("grid16x21_bf16_l2_k4x2", "bf16", 2, (4, 2), 21, height=16), _CMP),  # padded
    (_grid("rect60x80_bf16_l3_k8x4x2", "bf16", 3, (8, 4, 2), 80, height=60), _CMP | _SIZE),
    (_grid("grid64_bf16_l2_k4_d128", "bf16", 2, 4, 64, d=128), _CMP),
    (synth.WORKLOADS["grid128_bf16_l2_k16"], _CMP),
]


@pytest.mark.parametrize("w,flags", _COMPLEMENT,
                         ids=["%s_f%d" % (w.name, f) for w, f in _COMPLEMENT])
def test_complement_enrichment(w, flags):
    _full_check(w, flags=flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_complement_with_zero_queries_averages_every_token(dtype):
    """Q = 0 with the complement and size-weighted logits: the fine tokens and
    the unpicked candidates' pooled tokens cover every key token once, so
    every output is the mean of all N values and lse = ln N (a closed form,
    independent of the oracle)."""
    w = small("zeroq_cmp", 1, 2, 64, dtype, 2, 4)
    inp = synth.make_inputs(w)
    inp["q"] = np.zeros_like(inp["q"])
    inp["q64"] = np.zeros_like(inp["q64"])
    gpu = gpu_run(w, inp, flags=_CMP | _SIZE, backward=False)
    z = oracle_inputs(w, inp)
    want = np.broadcast_to(z["v"].mean(axis=1, keepdims=True), z["v"].shape)
    tol = TOL[dtype]
    assert_close(gpu["out"], want, tol["out_max"], tol["out_mean"], "out")
    assert_close(gpu["lse"], np.full_like(gpu["lse"], np.log(w.N)), tol["out_max"], what="lse")


# head dimension 128 (the one-block bf16 kernels and the fp32 kernels)
_D128 = [
    (_grid("grid32_f32_l1_k8_d128", "f32", 1, 8, 32, H=1, d=128), 0),
    (_grid("grid32_f32_l2_k2_d128", "f32", 2, 2, 32, d=128), oracle.SIZE_BIAS),
    (_grid("grid64_bf16_l1_k16_d128", "bf16", 1, 16, 64, d=128), 0),
    (_grid("grid64_bf16_l2_k4_d128", "bf16", 2, 4, 64, d=128), 0),
    (_grid("grid64_bf16_l2_k4_d128", "bf16", 2, 4, 64, d=128),
     oracle.ENRICH_COARSE | oracle.SIZE_BIAS),
    (_grid("grid64_bf16_l3_k1_d128", "bf16", 3, 1, 64, d=128), 0),
    (_grid("grid64_bf16_l2_k8x4_d128", "bf16", 2, (8, 4), 64, d=128), 0),
    (_grid("rect48x80_bf16_l2_k8_d128", "bf16", 2, 8, 80, height=48, d=128), oracle.NO_ENRICH),
]


@pytest.mark.parametrize("w,flags", _D128, ids=["%s_f%d" % (w.name, f) for w, f in _D128])
def test_head_dim_128(w, flags):
    _full_check(w, flags=flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_blocks_no_enrichment_equals_dense(dtype):
    """Every key block selected, enrichment off: the method is dense softmax
    attention, so out, lse and the gradients are the closed forms of dense
    attention (written out here in numpy, independently of the oracle):
    P = softmax(s Q K^T), O = P V, dV = P^T dO, dS = P o (dO V^T - rowsum(dO o O)),
    dQ = s dS K, dK = s dS^T Q."""
    w = small("dense", 1, 2, 32, dtype, 1, 64)  # K = n_1 = 64: every block
    inp = synth.make_inputs(w)
    gpu = gpu_run(w, inp, flags=oracle.NO_ENRICH)
    z = oracle_inputs(w, inp)
    s = 1.0 / np.sqrt(w.d)
    q, k, v, do = z["q"], z["k"], z["v"], z["do"]
    logits = s * (q @ k.transpose(0, 2, 1))
    m = logits.max(2, keepdims=True)
    p = np.exp(logits - m)
    p_sum = p.sum(2, keepdims=True)
    P = p / p_sum
    want = P @ v
    lse = (m + np.log(p_sum))[..., 0]
    dv = P.transpose(0, 2, 1) @ do
    dS = P * (do @ v.transpose(0, 2, 1) - (do * want).sum(2, keepdims=True))
    dq = s * (dS @ k)
    dk = s * (dS.transpose(0, 2, 1) @ q)
    tol = TOL[dtype]
    assert_close(gpu["out"], want, tol["out_max"], tol["out_mean"], "out")
    assert_close(gpu["lse"], lse, tol["out_max"], tol["out_mean"], "lse")
    for n_, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(gpu[n_], ref, tol["grad_max"], what=n_)


@pytest.mark.parametrize("w", [small("peak_f32", 1, 2, 32, "f32", 2, 2),
                               small("peak_bf16", 1, 2, 64, "bf16", 2, 4)],
                         ids=lambda w: w.name)
def test_peaked_logits(w):
    """Q and K scaled by 4 (exactly: a power of two), so logits spread over
    about +-50 and most softmax weights underflow: the online softmax's
    running maximum moves far more often than on unit-scale inputs.  Out
    keeps its tolerance (it is still a convex combination of V rows).  lse
    grows with the logits (here to about 50, where one fp32 ulp is 3.8e-6 and
    a 64-term fp32 dot product may be off by several), so on fp32 its bound
    is out_max relative to its largest magnitude; on bf16 the absolute 2e-2
    already covers it.  The gradients grow with Q and K (here to about 16 in
    magnitude) and every rounding on the bf16 path is relative to the values
    it rounds, so their bound is grad_tol's: 5e-2, or 2^-6 of the tensor's
    largest magnitude when that is larger (fp32: 1e-4 relative to that
    magnitude)."""
    inp = synth.make_inputs(w)
    for n_ in ("q", "k"):
        inp[n_], inp[n_ + "64"] = synth._cast(inp[n_ + "64"] * 4.0, w.dtype)
        assert np.array_equal(inp[n_ + "64"] / 4.0, synth.make_inputs(w)[n_ + "64"])
    gpu = gpu_run(w, inp)
    z = oracle_inputs(w, inp)
    tol = TOL[w.dtype]
    qp, kp, vp = (oracle.pool(z[n_], BS, w.levels) for n_ in ("q", "k", "v"))
    check_selection(w, gpu, (qp, kp), exact=(w.dtype == "f32"))
    idx = gpu["idx"]
    scale = 1.0 / np.sqrt(w.d)
    o, lse = oracle.forward(z["q"], z["k"], z["v"], kp, vp, idx, BS, scale)
    assert_close(gpu["out"], o, tol["out_max"], tol["out_mean"], "out")
    lse_scale = max(1.0, float(np.abs(lse).max())) if w.dtype == "f32" else 1.0
    assert_close(gpu["lse"], lse, tol["out_max"] * lse_scale, tol["out_mean"] * lse_scale, "lse")
    dq, dk, dv = oracle.backward(z["q"], z["k"], z["v"], kp, vp, idx, o, lse, z["do"], BS, scale)
    for n_, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        bound = (grad_tol(ref, tol["grad_max"]) if w.dtype == "bf16"
                 else tol["grad_max"] * max(1.0, float(np.abs(ref).max())))
        assert_close(gpu[n_], ref, bound, what=n_)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_query_ties_resolve_to_lowest_blocks(dtype):
    w = small("zeroq", 1, 2, 64, dtype, 2, 4)
    inp = synth.make_inputs(w)
    inp["q"] = np.zeros_like(inp["q"])
    inp["q64"] = np.zeros_like(inp["q64"])
    gpu = gpu_run(w, inp)
    for lvl in gpu["idx"]:
        assert np.all(lvl == np.arange(w.topk)[None, None, :])
    n_ent = BS * w.topk + w.levels * w.topk
    np.testing.assert_allclose(gpu["lse"], np.log(n_ent), rtol=0, atol=1e-5)
    check_transpose(gpu, w)  # degenerate lists: blocks 0..K-1 hold every row
    # values and gradients on these lists: uniform weights over every entry
    z = oracle_inputs(w, inp)
    qp, kp, vp = (oracle.pool(z[n_], BS, w.levels) for n_ in ("q", "k", "v"))
    o, lse, dq, dk, dv = oracle_values(w, z, kp, vp, gpu["idx"])
    tol = TOL[dtype]
    assert_close(gpu["out"], o, tol["out_max"], tol["out_mean"], "out")
    for n_, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(gpu[n_], ref, tol["grad_max"], what=n_)
    # keys outside blocks 0..K-1 (and their pooled parents) are never attended
    assert np.all(gpu["dv"][:, BS * w.topk * BS ** (w.levels - 1):] == 0)


def test_runs_are_bit_identical():
    import torch
    w = small("det", 1, 2, 64, "bf16", 2, 4)
    inp = synth.make_inputs(w)
    a = gpu_run(w, inp)
    b = gpu_run(w, inp)
    for n_ in ("out_t", "lse_t", "dq_t", "dk_t", "dv_t"):
        assert torch.equal(a[n_].view(torch.int16) if a[n_].dtype == torch.bfloat16 else a[n_],
                           b[n_].view(torch.int16) if b[n_].dtype == torch.bfloat16 else b[n_]), n_
    for l in range(w.levels):
        np.testing.assert_array_equal(a["idx"][l], b["idx"][l])
        np.testing.assert_array_equal(a["col"][l], b["col"][l])


def test_repeated_parts_keep_the_transpose_exact():
    """Stages may be re-run on the same workspace (here: selection three times,
    transpose twice): the key->query lists stay the exact transpose of the
    index lists and the gradients do not change."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    w = small("rep", 1, 2, 64, "bf16", 2, 4)
    inp = synth.make_inputs(w)
    a = gpu_run(w, inp)
    B, H, N, d = w.B, w.H, w.N, w.d
    ws = a["ws"]
    do = to_device(inp["do"], w.dtype)
    dq, dk, dv = (torch.empty_like(a["q"]) for _ in range(3))
    args = (B, H, N, d, BS, w.topk, w.levels, lib.BF16, 0, ws, ws.numel())
    for _ in range(3):
        lib.llsa_forward_part(lib.PART_SELECT, a["q"], a["k"], a["v"], a["out_t"], a["lse_t"], *args)
    for _ in range(2):
        lib.llsa_backward_part(lib.PART_TRANSPOSE, a["q"], a["k"], a["v"], a["out_t"], a["lse_t"],
                               do, dq, dk, dv, *args)
    for part in (lib.PART_DQ, lib.PART_ENRICH, lib.PART_DKDV):
        lib.llsa_backward_part(part, a["q"], a["k"], a["v"], a["out_t"], a["lse_t"], do, dq, dk, dv,
                               *args)
    torch.cuda.synchronize()
    G = B * H
    for l in range(w.levels):
        n = N // BS ** (l + 1)
        rp = ws_array(ws, a["lay"]["rowptr"][l], G * (n + 1), np.int32).reshape(G, n + 1)
        col = ws_array(ws, a["lay"]["col"][l], G * n * w.topk, np.int32).reshape(G, n * w.topk)
        want_rp, want_col = oracle.transpose(a["idx"][l])
        np.testing.assert_array_equal(rp, want_rp)
        np.testing.assert_array_equal(col, want_col)
    for got, ref in ((dq, a["dq_t"]), (dk, a["dk_t"]), (dv, a["dv_t"])):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_whole_calls_on_a_side_stream_match_stage_order():
    """On a caller stream other than the default one, two back-to-back
    llsa_forward + llsa_backward calls with different inputs and workspaces
    (no host sync between them) give, bit for bit, the output, gradients and
    key->query lists of the stage-by-stage part sequence on the default stream
    (llsa_forward lets its pool launch zero the pick counters; the selection
    part on its own zeroes them itself)."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    ws_ = [small("side%d" % s_, 1, 3, 128, "bf16", 2, 8, seed=s_) for s_ in (1, 2)]
    dev = []
    for w in ws_:
        inp = synth.make_inputs(w)
        q, k, v = (to_device(inp[n_], "bf16").reshape(w.B, w.H, w.N, w.d) for n_ in "qkv")
        do = to_device(inp["do"], "bf16").reshape(w.B, w.H, w.N, w.d)
        dev.append((w, q, k, v, do))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = []
    with torch.cuda.stream(side):
        for w, q, k, v, do in dev:
            out, lse, ws = lib.forward(q, k, v, w.topk, w.levels)
            got.append((out, lse, ws) + lib.backward(q, k, v, out, lse, do, w.topk, w.levels, ws))
    side.synchronize()
    for (w, q, k, v, do), (out, lse, ws, dq, dk, dv) in zip(dev, got):
        args = (w.B, w.H, w.N, w.d, BS, w.topk, w.levels, lib.BF16, 0)
        ws2 = torch.empty_like(ws)
        out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
        dq2, dk2, dv2 = (torch.empty_like(q) for _ in range(3))
        for part in (lib.PART_POOL, lib.PART_SELECT, lib.PART_ATTN):
            lib.llsa_forward_part(part, q, k, v, out2, lse2, *args, ws2, ws2.numel())
        for part in (lib.PART_TRANSPOSE, lib.PART_DQ, lib.PART_ENRICH, lib.PART_DKDV):
            lib.llsa_backward_part(part, q, k, v, out2, lse2, do, dq2, dk2, dv2, *args, ws2,
                                   ws2.numel())
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
            assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
        lay = lib.llsa_workspace_layout_lk(w.B, w.H, w.N, w.d, BS, [w.topk] * w.levels,
                                           w.levels, lib.BF16)
        G = w.B * w.H
        for l in range(w.levels):
            n = w.N // BS ** (l + 1)
            for off, cnt in ((lay["rowptr"][l], G * (n + 1)), (lay["col"][l], G * n * w.topk)):
                np.testing.assert_array_equal(ws_array(ws, off, cnt, np.int32),
                                              ws_array(ws2, off, cnt, np.int32))


def test_whole_calls_on_a_reused_garbage_workspace():
    """llsa_forward zeroes the selection's pick counters itself (in its pool
    launch): a workspace filled with 0xFF bytes, then reused by a second
    forward + backward, gives bit for bit the results of a fresh one, and the
    key->query lists stay the exact transpose of the index lists."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    w = small("reuse", 1, 2, 64, "bf16", 2, 4)
    inp = synth.make_inputs(w)
    q, k, v, do = (to_device(inp[n_], "bf16") for n_ in ("q", "k", "v", "do"))
    out0, lse0, ws0 = lib.forward(q, k, v, w.topk, w.levels)
    ref = (out0,) + lib.backward(q, k, v, out0, lse0, do, w.topk, w.levels, ws0)
    ws = torch.full_like(ws0, 255)
    G = w.B * w.H
    lay = lib.llsa_workspace_layout_lk(w.B, w.H, w.N, w.d, BS, [w.topk] * w.levels, w.levels,
                                       lib.BF16)
    for _ in range(2):
        out, lse, _ws = lib.forward(q, k, v, w.topk, w.levels, workspace=ws)
        got = (out,) + lib.backward(q, k, v, out, lse, do, w.topk, w.levels, ws)
        torch.cuda.synchronize()
        for a_, b_ in zip(got, ref):
            assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
        for l in range(w.levels):
            n = w.N // BS ** (l + 1)
            idx = ws_array(ws, lay["idx"][l], G * n * w.topk, np.int32).reshape(G, n, w.topk)
            rp = ws_array(ws, lay["rowptr"][l], G * (n + 1), np.int32).reshape(G, n + 1)
            col = ws_array(ws, lay["col"][l], G * n * w.topk, np.int32).reshape(G, n * w.topk)
            want_rp, want_col = oracle.transpose(idx)
            np.testing.assert_array_equal(rp, want_rp)
            np.testing.assert_array_equal(col, want_col)


# ------------------------------------------------------- full-size workloads

def _needed_qblocks(w, idx, kblocks):
    """Query blocks whose tokens feed dk/dv of the given key blocks."""
    need = set()
    for l in range(1, w.levels + 1):
        for j in kblocks:
            a = j // BS ** (l - 1)
            hits = np.nonzero(np.any(idx[l - 1][0] == a, axis=1))[0]
            for b in hits:
                need.update(range(b * BS ** (l - 1), (b + 1) * BS ** (l - 1)))
    return np.array(sorted(need), dtype=np.int64)


# every head, block and token compared, in the benchmark's launch
# configuration; the oracle runs one head per host thread
_FULL = [synth.WORKLOADS[n] for n in (
    "grid128_bf16_l2_k16", "grid256_bf16_l2_k16", "grid512_bf16_l3_k16",
    "video16x64x64_bf16_l2_k16", "rect192x320_bf16_l2_k16",
    "grid256_d128_bf16_l2_k16")] + [
    # coarsest levels of 1024 and 480 blocks under a finer level: the fused
    # two-level selection with 16 keys per lane in its first phase
    _grid("grid512_bf16_l2_k16", "bf16", 2, 16, 512, H=2),
    _grid("rect384x320_bf16_l2_k24", "bf16", 2, 24, 320, height=384, H=1, d=128),
    # the deepest pyramids N <= 2^23 allows: 4 and 5 levels down to one block
    _grid("grid256_bf16_l4_k1", "bf16", 4, 1, 256, H=1),
    _grid("grid1024_bf16_l5_k1", "bf16", 5, 1, 1024, H=1),
    # 200 x 200 (N = 40000): 2500 level-1 and 157 level-2 blocks, the last
    # of which covers 4 level-1 blocks
    _grid("rect200x200_bf16_l2_k16", "bf16", 2, 16, 200, height=200, H=6, sigma=4.0),
]


@pytest.mark.parametrize("w", _FULL, ids=lambda w: w.name)
def test_full_size(w):
    """Full-size workloads: pyramid, selection, transposes, out, lse and
    every gradient against the oracle, element by element, all heads."""
    _full_check(w)


@pytest.mark.parametrize("w", [synth.WORKLOADS["grid256_bf16_l2_k16"]], ids=lambda w: w.name)
def test_full_size_complement(w):
    """The complement variant at 256 x 256 (496 pooled entries per query
    block), element by element, all heads."""
    _full_check(w, flags=oracle.ENRICH_COMPLEMENT)


# the largest N the boundary accepts (2^23 tokens, 1 GiB per head and
# tensor), two heads; white inputs keep the generator fast.  The oracle would
# need minutes per head here, so outputs and gradients are compared on
# sampled blocks
_SAMPLED = [_grid("rect2048x4096_bf16_l3_k16", "bf16", 3, 16, 4096, height=2048, H=2, sigma=0.0)]


@pytest.mark.parametrize("w", _SAMPLED, ids=lambda w: w.name)
def test_full_size_sampled(w):
    """The largest workload: pyramid, selection and transposes checked in
    full; outputs and gradients on 128 sampled query blocks and 8 key blocks
    of every head (the oracle computes them one by one)."""
    from llsa_check import per_head
    inp = synth.make_inputs(w)
    gpu = gpu_run(w, inp)
    z = oracle_inputs(w, inp)
    qp, kp, vp = (oracle.pool(z[n], BS, w.levels) for n in ("q", "k", "v"))
    for l in range(w.levels):
        assert_close(gpu["kbar"][l], kp[l], 2e-6, what="kbar level %d" % (l + 1))
    check_selection(w, gpu, (qp, kp), exact=False)
    check_transpose(gpu, w)
    tol = TOL[w.dtype]
    n1 = w.N // BS
    scale = 1.0 / np.sqrt(w.d)

    def head(h):
        rng = np.random.default_rng(1 + h)
        sl = slice(h, h + 1)
        q0, k0, v0, do0 = (z[n][sl] for n in ("q", "k", "v", "do"))
        kp0, vp0 = [x[sl] for x in kp], [x[sl] for x in vp]
        idx0 = [x[sl] for x in gpu["idx"]]
        qbl = np.sort(rng.choice(n1, 128, replace=False))
        # key blocks inside one top-level block keep the oracle's work bounded
        top = BS ** (w.levels - 1)
        j0 = int(rng.integers(0, n1 // top)) * top
        kbl = np.sort(rng.choice(np.arange(j0, j0 + top), min(8, top), replace=False))
        rows = np.union1d(qbl, _needed_qblocks(w, idx0, kbl))
        o, lse = oracle.forward(q0, k0, v0, kp0, vp0, idx0, BS, scale, qblocks=rows)
        dq, dk, dv = oracle.backward(q0, k0, v0, kp0, vp0, idx0, o, lse, do0, BS, scale,
                                     qblocks=qbl, kblocks=kbl)
        tok = (qbl[:, None] * BS + np.arange(BS)).ravel()
        ktok = (kbl[:, None] * BS + np.arange(BS)).ravel()
        return (o[0, tok], lse[0, tok], dq[0, tok], dk[0, ktok], dv[0, ktok], tok, ktok)

    for h, (o, lse, dq, dk, dv, tok, ktok) in enumerate(per_head(head, w.G)):
        assert_close(gpu["out"][h, tok], o, tol["out_max"], tol["out_mean"], "out")
        assert_close(gpu["lse"][h, tok], lse, tol["out_max"], tol["out_mean"], "lse")
        assert_close(gpu["dq"][h, tok], dq, tol["grad_max"], what="dq")
        assert_close(gpu["dk"][h, ktok], dk, tol["grad_max"], what="dk")
        assert_close(gpu["dv"][h, ktok], dv, tol["grad_max"], what="dv")
