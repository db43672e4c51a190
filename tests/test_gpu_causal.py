"""GPU parity of the causal variant (CAUSAL): token t attends keys u <= t.

The README's usage names the non-causal form only; the reading taken (the
oracle's ORC_CAUSAL): at every level a query block keeps its own block and
its best K-1 earlier candidates (-1 in the slots left), the own fine block is
masked to keys u <= t, and no ancestor's own pooled token enriches.

Checks: every stage against the oracle (the selection by the gap rule on
bf16); dense causal attention in closed form when every earlier block is
picked and nothing enriches; and, at the headline size, that the outputs of
tokens before a cut are bit for bit unchanged by any change of the keys and
values after it, and the key gradients after a cut by any change of the
queries and output gradients before it.
"""
import numpy as np
import pytest

import oracle
import synth
from llsa_check import BS, TOL, assert_close, full_check, gpu_run, oracle_inputs, to_device

pytestmark = pytest.mark.gpu

W = synth.Workload
C = oracle.CAUSAL
_SIZE, _COARSE, _NONE = oracle.SIZE_BIAS, oracle.ENRICH_COARSE, oracle.NO_ENRICH


def _w(name, dtype, L, K, side, height=0, B=1, H=2, d=64, sigma=2.0):
    return W(name, B, H, side, d, dtype, L, K, sigma, 0, 16, 1, height)


_CASES = [
    (synth.WORKLOADS["grid32_f32_l1_k8"], C),
    (_w("grid32_f32_l2_k2", "f32", 2, 2, 32), C),
    (_w("grid32_f32_l2_k4", "f32", 2, 4, 32), C | _SIZE),
    (_w("grid16_bf16_l1_k4", "bf16", 1, 4, 16, H=3), C),
    (_w("grid32_bf16_l2_k2", "bf16", 2, 2, 32, B=2, H=1), C),
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), C),
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), C | _SIZE),
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), C | _COARSE),
    (_w("grid64_bf16_l2_k4", "bf16", 2, 4, 64), C | _NONE),
    (_w("grid64_bf16_l2_k5x3", "bf16", 2, (5, 3), 64), C),            # odd fine count
    (_w("grid64_bf16_l3_k1", "bf16", 3, 1, 64), C),                   # the block itself only
    (_w("grid64_bf16_l1_k32", "bf16", 1, 32, 64, H=1), C),
    (synth.WORKLOADS["grid64_bf16_l1_k16"], C),                       # the four-block shape
    (_w("grid16x21_bf16_l2_k4x2", "bf16", 2, (4, 2), 21, height=16), C),   # N = 336
    (_w("grid16x21_f32_l2_k4x2", "f32", 2, (4, 2), 21, height=16), C),
    (_w("rect60x80_bf16_l3_k8x4x2", "bf16", 3, (8, 4, 2), 80, height=60), C | _SIZE),
    (_w("grid64_bf16_l2_k4_d128", "bf16", 2, 4, 64, d=128), C),
    (_w("grid64_f32_l2_k4_d128", "f32", 2, 4, 64, d=128, H=1), C),
    (synth.WORKLOADS["grid128_bf16_l2_k16"], C),
]


@pytest.mark.parametrize("w,flags", _CASES, ids=["%s_f%d" % (w.name, f) for w, f in _CASES])
def test_causal_against_the_oracle(w, flags):
    gpu = full_check(w, flags=flags)
    # every row keeps its own block
    for l, idx in enumerate(gpu["idx"], 1):
        rows = np.arange(idx.shape[1])[None, :, None]
        assert np.all(np.any(idx == rows, axis=2)), "level %d" % l


def test_causal_full_size():
    full_check(synth.WORKLOADS["grid256_bf16_l2_k16"], flags=C)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,K", [(1, 64), (2, (64, 4))])
def test_every_earlier_block_equals_dense_causal(dtype, L, K):
    """Every earlier block picked, no enrichment: dense causal softmax
    attention, written out here in numpy (independently of the oracle)."""
    w = _w("dense_causal", dtype, L, K, 32)  # n1 = 64, n2 = 4
    inp = synth.make_inputs(w)
    gpu = gpu_run(w, inp, flags=C | _NONE)
    z = oracle_inputs(w, inp)
    s = 1.0 / np.sqrt(w.d)
    q, k, v, do = z["q"], z["k"], z["v"], z["do"]
    N = w.N
    logits = np.where(np.tril(np.ones((N, N), bool)), s * (q @ k.transpose(0, 2, 1)), -np.inf)
    m = logits.max(2, keepdims=True)
    p = np.exp(logits - m)
    P = p / p.sum(2, keepdims=True)
    want = P @ v
    lse = (m + np.log(p.sum(2, keepdims=True)))[..., 0]
    dS = P * (do @ v.transpose(0, 2, 1) - (do * want).sum(2, keepdims=True))
    tol = TOL[dtype]
    assert_close(gpu["out"], want, tol["out_max"], tol["out_mean"], "out")
    assert_close(gpu["lse"], lse, tol["out_max"], tol["out_mean"], "lse")
    for n_, ref in (("dq", s * dS @ k), ("dk", s * dS.transpose(0, 2, 1) @ q),
                    ("dv", P.transpose(0, 2, 1) @ do)):
        assert_close(gpu[n_], ref, tol["grad_max"], what=n_)


def _tokens(shape, seed, dtype):
    st, _ = synth.random_tensor(shape, seed, dtype)
    return to_device(st, dtype)


@pytest.mark.parametrize("flags", [C, C | _SIZE])
def test_later_keys_do_not_reach_earlier_outputs(flags):
    """Headline shape (256^2 tokens, two levels, top-16, bf16), tokens in
    attention order: keys and values after a cut t0 replaced by fresh noise
    leave out and lse of every token <= t0 bit for bit unchanged."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    B, H, N, d = 1, 6, 65536, 64
    q, k, v = (_tokens((B, H, N, d), s, "bf16") for s in (1, 2, 3))
    out0, lse0, _ = lib.forward(q, k, v, 16, 2, flags)
    for t0 in (4095, 30000, 65534):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, t0 + 1:] = _tokens((B, H, N - t0 - 1, d), 10 + t0 % 7, "bf16")
        v2[:, :, t0 + 1:] = _tokens((B, H, N - t0 - 1, d), 20 + t0 % 7, "bf16")
        out1, lse1, _ = lib.forward(q, k2, v2, 16, 2, flags)
        torch.cuda.synchronize()
        assert torch.equal(out1[:, :, :t0 + 1], out0[:, :, :t0 + 1]), t0
        assert torch.equal(lse1[:, :, :t0 + 1], lse0[:, :, :t0 + 1]), t0
        assert not torch.equal(out1, out0)


def test_earlier_queries_do_not_reach_later_key_gradients():
    """Headline shape: queries and output gradients before a cut T0 (a
    multiple of 16^2, so no block straddles it) replaced by fresh noise leave
    dk, dv of every key >= T0, and dq of every query >= T0, bit for bit
    unchanged (a query attends only keys at or before it)."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    B, H, N, d = 1, 6, 65536, 64
    q, k, v, do = (_tokens((B, H, N, d), s, "bf16") for s in (4, 5, 6, 7))

    def grads(q_, do_):
        out, lse, ws = lib.forward(q_, k, v, 16, 2, C)
        return lib.backward(q_, k, v, out, lse, do_, 16, 2, ws, C)

    dq0, dk0, dv0 = grads(q, do)
    for T0 in (256, 32768, 65280):
        q2, do2 = q.clone(), do.clone()
        q2[:, :, :T0] = _tokens((B, H, T0, d), 30 + T0 % 5, "bf16")
        do2[:, :, :T0] = _tokens((B, H, T0, d), 40 + T0 % 5, "bf16")
        dq1, dk1, dv1 = grads(q2, do2)
        torch.cuda.synchronize()
        for a, b_, name in ((dk1, dk0, "dk"), (dv1, dv0, "dv"), (dq1, dq0, "dq")):
            assert torch.equal(a[:, :, T0:], b_[:, :, T0:]), (name, T0)
        assert not torch.equal(dk1, dk0)
