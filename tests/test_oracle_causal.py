"""Pins of the causal variant (ORC_CAUSAL, reading R24).

The README's usage note says the implementation is non-causal only.  Reading
taken: token t attends keys u <= t; at every level the query's ancestor block
keeps itself and its best K-1 earlier candidates (all of them if fewer; -1 in
the slots left); the diagonal fine block is masked to keys u <= t; an
ancestor's own pooled token (its mean holds later tokens) does not enrich.

Pins: brute-force selection; with every earlier block picked and no
enrichment, dense causal attention; changing any key or value after t leaves
o_t bit for bit unchanged; the transpose of lists with unused slots against
a dense mask; finite differences.
"""
import numpy as np
import pytest

import oracle

BS = 16
CAUSAL = oracle.CAUSAL


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute_causal_select(qp, kp, K, N, L, scale):
    ks = oracle.level_topk(K, L)
    n = oracle.level_sizes(N, BS, L)
    idx = [None] * L
    for l in range(L, 0, -1):
        G = qp[l - 1].shape[0]
        out = np.full((G, n[l - 1], ks[l - 1]), -1, np.int32)
        for g in range(G):
            for i in range(n[l - 1]):
                if l == L:
                    cand = np.arange(i)
                else:
                    par = [c for c in idx[l][g, i // BS] if c >= 0]
                    cand = np.array([BS * c + r for c in par for r in range(BS)
                                     if BS * c + r < min(i, n[l - 1])], dtype=np.int64)
                keep = []
                if len(cand):
                    sc = scale * kp[l - 1][g, cand] @ qp[l - 1][g, i]
                    keep = list(cand[np.lexsort((cand, -sc))[:ks[l - 1] - 1]])
                row = sorted(keep + [i])
                out[g, i, :len(row)] = row
        idx[l - 1] = out
    return idx


@pytest.mark.parametrize("N,L,K", [(256, 1, 4), (1024, 2, (3, 2)), (4096, 2, (8, 4)),
                                   (336, 2, (4, 2)), (16384, 3, (2, 3, 2))])
def test_selection_matches_brute_force(N, L, K):
    q, k = _rand((2, N, 8), 1), _rand((2, N, 8), 2)
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    got, _ = oracle.select(qp, kp, K, BS, 0.3, N=N, causal=True)
    want = _brute_causal_select(qp, kp, K, N, L, 0.3)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)
    # every row keeps its own block; earlier rows hold -1 in the slots left
    for l, a in enumerate(got, 1):
        rows = np.arange(a.shape[1])
        assert np.all(np.any(a == rows[None, :, None], axis=2))
        assert np.all((a < 0) | (a <= rows[None, :, None]))


def _dense_causal(q, k, v, s):
    G, N, d = q.shape
    z = s * q @ k.transpose(0, 2, 1)
    z = np.where(np.tril(np.ones((N, N), bool))[None], z, -np.inf)
    m = z.max(2, keepdims=True)
    p = np.exp(z - m)
    return (p / p.sum(2, keepdims=True)) @ v, (m + np.log(p.sum(2, keepdims=True)))[..., 0], p / p.sum(2, keepdims=True)


@pytest.mark.parametrize("N,L,K", [(1024, 1, 64), (1024, 2, (64, 4)), (336, 2, (32, 2))])
def test_every_earlier_block_picked_equals_dense_causal(N, L, K):
    G, d = 1, 8
    q, k, v, do = (_rand((G, N, d), s) for s in (3, 4, 5, 6))
    s = 1.0 / np.sqrt(d)
    r = oracle.run(q, k, v, BS, L, K, flags=CAUSAL | oracle.NO_ENRICH, dout=do)
    o, lse, P = _dense_causal(q, k, v, s)
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)
    dS = P * (do @ v.transpose(0, 2, 1) - (do * o).sum(2, keepdims=True))
    np.testing.assert_allclose(r["dv"], P.transpose(0, 2, 1) @ do, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dq"], s * dS @ k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dk"], s * dS.transpose(0, 2, 1) @ q, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,L,K,flags", [(1024, 2, (4, 2), 0), (4096, 2, (8, 4), oracle.SIZE_BIAS),
                                         (336, 2, (4, 2), 0), (4096, 3, (4, 2, 1), 0),
                                         (1024, 2, (4, 2), oracle.ENRICH_COARSE)])
def test_later_keys_and_values_do_not_reach_earlier_outputs(N, L, K, flags):
    G, d = 2, 8
    q, k, v = (_rand((G, N, d), s) for s in (7, 8, 9))
    r0 = oracle.run(q, k, v, BS, L, K, flags=flags | CAUSAL)
    rng = np.random.default_rng(10)
    for cut in (0, 5, 16 * 7 + 3, N // 2 + 1, N - 2):
        k2, v2 = k.copy(), v.copy()
        k2[:, cut + 1:] += rng.standard_normal(k2[:, cut + 1:].shape) * 3
        v2[:, cut + 1:] += rng.standard_normal(v2[:, cut + 1:].shape) * 3
        r1 = oracle.run(q, k2, v2, BS, L, K, flags=flags | CAUSAL)
        np.testing.assert_array_equal(r1["out"][:, :cut + 1], r0["out"][:, :cut + 1])
        np.testing.assert_array_equal(r1["lse"][:, :cut + 1], r0["lse"][:, :cut + 1])


def test_transpose_skips_unused_slots():
    q, k = _rand((2, 1024, 8), 11), _rand((2, 1024, 8), 12)
    qp, kp = oracle.pool(q, BS, 2), oracle.pool(k, BS, 2)
    idx, _ = oracle.select(qp, kp, (4, 2), BS, 0.3, causal=True)
    for I in idx:
        G, n, K = I.shape
        rp, col = oracle.transpose(I)
        mask = np.zeros((G, n, n), bool)  # [g, query block, key block]
        for g in range(G):
            for i in range(n):
                for j in I[g, i]:
                    if j >= 0:
                        mask[g, i, j] = True
        for g in range(G):
            assert rp[g, -1] == mask[g].sum()
            for j in range(n):
                np.testing.assert_array_equal(col[g, rp[g, j]:rp[g, j + 1]],
                                              np.nonzero(mask[g, :, j])[0])


@pytest.mark.parametrize("N,L,K,flags", [(256, 1, 4, 0), (1024, 2, (3, 2), 0),
                                         (1024, 2, (3, 2), oracle.SIZE_BIAS), (336, 2, (4, 2), 0)])
def test_finite_differences(N, L, K, flags):
    G, d = 1, 8
    rng = np.random.default_rng(N + flags + 1)
    q, k, v, do = (rng.standard_normal((G, N, d)) for _ in range(4))
    fl = flags | CAUSAL
    r = oracle.run(q, k, v, BS, L, K, flags=fl, dout=do)
    grads = {"q": r["dq"], "k": r["dk"], "v": r["dv"]}
    eps = 1e-6
    checked = total = 0
    for name in ("q", "k", "v"):
        coords = [(0, int(t), int(c)) for t, c in zip(rng.integers(0, N, 40),
                                                       rng.integers(0, d, 40))]
        total += len(coords)
        for co in coords:
            vals, flipped = [], False
            for sgn in (1, -1):
                args = {"q": q, "k": k, "v": v}
                x = args[name].copy()
                x[co] += sgn * eps
                args[name] = x
                rr = oracle.run(args["q"], args["k"], args["v"], BS, L, K, flags=fl)
                flipped |= any(not np.array_equal(a, b) for a, b in zip(rr["idx"], r["idx"]))
                vals.append(float((rr["out"] * do).sum()))
            if flipped:
                continue
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grads[name][co]) <= 1e-6 * max(1.0, abs(fd)), (name, co, fd,
                                                                          grads[name][co])
            checked += 1
    assert checked >= 0.9 * total
