"""Pins of the oracle's backward pass.

The pages state that LLSA is trainable and runs its sparse kernels in both the
forward and the backward pass (page 2, summary and "Core Technique" 3), but
print no gradient formula.  The oracle's gradient is pinned to finite
differences of its own forward (selection held fixed, since Top-K is piecewise
constant) and, with every block selected and no enrichment, to the closed-form
gradient of dense softmax attention.
"""
import numpy as np
import pytest

import oracle

BS = 16


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss_and_idx(q, k, v, dout, L, K, flags):
    r = oracle.run(q, k, v, BS, L, K, flags=flags)
    return float((r["out"] * dout).sum()), r["idx"]


@pytest.mark.parametrize("N,L,K,flags", [(256, 1, 4, 0), (256, 1, 4, oracle.NO_ENRICH),
                                         (1024, 2, 2, 0), (256, 1, 4, oracle.SIZE_BIAS),
                                         (1024, 2, 2, oracle.ENRICH_COARSE),
                                         (1024, 2, 2, oracle.ENRICH_COARSE | oracle.SIZE_BIAS),
                                         (1024, 2, (3, 2), 0),
                                         (1024, 2, (5, 1), oracle.SIZE_BIAS)])
def test_finite_differences(N, L, K, flags):
    G, d = 1, 8
    rng = np.random.default_rng(N + int(np.sum(K)) + flags)
    q, k, v, dout = (rng.standard_normal((G, N, d)) for _ in range(4))
    r = oracle.run(q, k, v, BS, L, K, flags=flags, dout=dout)
    grads = {"q": r["dq"], "k": r["dk"], "v": r["dv"]}
    eps = 1e-6
    skipped = checked = 0
    for name in ("q", "k", "v"):
        coords = [(0, int(t), int(c)) for t, c in zip(rng.integers(0, N, 60),
                                                       rng.integers(0, d, 60))]
        coords += [(0, t, c) for t in range(16) for c in range(0, d, 3)]
        for co in coords:
            args = {"q": q, "k": k, "v": v}
            vals = []
            flipped = False
            for sgn in (1, -1):
                x = args[name].copy()
                x[co] += sgn * eps
                a = dict(args, **{name: x})
                f, idx = _loss_and_idx(a["q"], a["k"], a["v"], dout, L, K, flags)
                flipped |= any(not np.array_equal(i0, i1) for i0, i1 in zip(idx, r["idx"]))
                vals.append(f)
            if flipped:
                skipped += 1
                continue
            fd = (vals[0] - vals[1]) / (2 * eps)
            an = grads[name][co]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, co, fd, an)
            checked += 1
    assert checked > 0.9 * (checked + skipped)


def test_dense_case_matches_closed_form_gradient():
    G, N, d = 2, 256, 8
    q, k, v, do = (_rand((G, N, d), s) for s in (21, 22, 23, 24))
    r = oracle.run(q, k, v, BS, 1, N // BS, flags=oracle.NO_ENRICH, dout=do)
    s = r["scale"]
    z = s * np.einsum("gtc,guc->gtu", q, k)
    p = np.exp(z - z.max(2, keepdims=True))
    p /= p.sum(2, keepdims=True)
    o = p @ v
    dp = do @ np.swapaxes(v, 1, 2)
    ds = p * (dp - (do * o).sum(2, keepdims=True))
    np.testing.assert_allclose(r["dq"], s * ds @ k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dk"], s * np.swapaxes(ds, 1, 2) @ q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dv"], np.swapaxes(p, 1, 2) @ do, rtol=0, atol=1e-12)


def test_enrichment_gradient_reaches_pooled_tokens():
    # With Q = 0 every token attends uniformly to blocks 0..K-1 and their pooled
    # tokens, so the value gradient is closed-form: each fine value of a
    # selected block gets sum_t dO_t / n_ent from the fine entry plus
    # sum_l (#tokens whose level-l ancestor selected it) / (n_ent * bs^l).
    G, N, d, L, K = 1, 4096, 4, 2, 2
    q = np.zeros((G, N, d))
    k, v, do = _rand((G, N, d), 30), _rand((G, N, d), 31), _rand((G, N, d), 32)
    r = oracle.run(q, k, v, BS, L, K, dout=do)
    n_ent = BS * K + L * K
    tot = do[0].sum(axis=0) / n_ent
    for x in range(N):
        want = np.zeros(d)
        if x // BS < K:
            want += tot                       # fine entry
            want += tot / BS                  # level-1 pooled entry
        if x // BS ** 2 < K:
            want += tot / BS ** 2             # level-2 pooled entry
        np.testing.assert_allclose(r["dv"][0, x], want, rtol=0, atol=1e-12)


def test_subsets_match_full():
    G, N, d = 1, 1024, 8
    q, k, v, do = (_rand((G, N, d), s) for s in (41, 42, 43, 44))
    r = oracle.run(q, k, v, BS, 2, 2, dout=do)
    qb, kb = [3, 40], [0, 7, 63]
    dq, dk, dv = oracle.backward(q, k, v, r["kpyr"], r["vpyr"], r["idx"], r["out"], r["lse"],
                                 do, BS, r["scale"], qblocks=qb, kblocks=kb)
    for i in qb:
        np.testing.assert_allclose(dq[:, BS * i:BS * (i + 1)], r["dq"][:, BS * i:BS * (i + 1)],
                                   rtol=0, atol=1e-13)
    for j in kb:
        sl = slice(BS * j, BS * (j + 1))
        np.testing.assert_allclose(dk[:, sl], r["dk"][:, sl], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[:, sl], r["dv"][:, sl], rtol=0, atol=1e-13)
