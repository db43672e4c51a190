"""Pins of the oracle where 16^levels does not divide the token count.

The README's usage limits the token count to powers of two and says later
versions will lift that limit (page 1, usage).  Reading taken: level l has
ceil(N / 16^l) blocks, block j covering tokens j 16^l .. min((j+1) 16^l, N) - 1
(the last block of a level may be partial -- the sequence is padded to a
multiple of 16^levels and the padding is never attended); a pooled token is
the mean of the tokens its block covers; a level's candidates are the blocks
that exist (below the coarsest level: the existing children of the parent's
picks); a pooled token passes 1/count of its gradient to each token it
averages.  Pins: plain slice means, brute-force selection, dense attention
(all blocks selected) with and without enrichment, the closed-form dense
gradient, and finite differences.
"""
import numpy as np
import pytest

import oracle

BS = 16


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _slice_means(x, span):
    """[G, N, d] -> means over consecutive runs of `span` tokens (last one partial)"""
    G, N, d = x.shape
    n = -(-N // span)
    return np.stack([x[:, j * span:min((j + 1) * span, N)].mean(axis=1) for j in range(n)], 1)


@pytest.mark.parametrize("N,L", [(100, 1), (336, 2), (1000, 2), (4100, 3), (256, 2)])
def test_pool_partial_blocks_are_means_of_their_tokens(N, L):
    x = _rand((2, N, 5), N)
    pyr = oracle.pool(x, BS, L)
    assert [p.shape[1] for p in pyr] == oracle.level_sizes(N, BS, L)
    for l in range(1, L + 1):
        np.testing.assert_allclose(pyr[l - 1], _slice_means(x, BS ** l), rtol=0, atol=1e-13)


def _brute_select(qp, kp, K, N, L, scale):
    """Top-K by sorting, level by level; candidates: existing blocks only."""
    ks = oracle.level_topk(K, L)
    n = oracle.level_sizes(N, BS, L)
    idx = [None] * L
    for l in range(L, 0, -1):
        G = qp[l - 1].shape[0]
        out = np.zeros((G, n[l - 1], ks[l - 1]), np.int32)
        for g in range(G):
            for i in range(n[l - 1]):
                if l == L:
                    cand = np.arange(n[l - 1])
                else:
                    par = idx[l][g, i // BS]
                    cand = np.array([BS * c + r for c in par for r in range(BS)
                                     if BS * c + r < n[l - 1]])
                sc = scale * kp[l - 1][g, cand] @ qp[l - 1][g, i]
                order = np.lexsort((cand, -sc))
                out[g, i] = np.sort(cand[order[:ks[l - 1]]])
        idx[l - 1] = out
    return idx


@pytest.mark.parametrize("N,L,K", [(336, 2, (4, 2)), (1000, 2, 3), (100, 1, 3),
                                   (4100, 3, (2, 2, 2)), (336, 2, (21, 2))])
def test_selection_matches_brute_force(N, L, K):
    q, k = _rand((2, N, 8), 1), _rand((2, N, 8), 2)
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    got, _ = oracle.select(qp, kp, K, BS, 0.3, N=N)
    want = _brute_select(qp, kp, K, N, L, 0.3)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)


def test_top_k_beyond_the_candidates_is_refused():
    # 336 tokens, two levels: the level-2 blocks cover 16 and 5 level-1 blocks,
    # so a level-1 row may have only 16 (2 - 1) + 5 = 21 candidates
    assert oracle.min_candidates(336, BS, 2, (21, 2)) == [21, 2]
    with pytest.raises(ValueError):
        oracle.check_topk(336, BS, 2, (22, 2))
    with pytest.raises(ValueError):
        oracle.check_topk(336, BS, 2, (4, 3))


def _dense(q, keys, vals, s):
    z = s * q @ keys.transpose(0, 2, 1)
    m = z.max(2, keepdims=True)
    p = np.exp(z - m)
    return (p / p.sum(2, keepdims=True)) @ vals, (m + np.log(p.sum(2, keepdims=True)))[..., 0]


@pytest.mark.parametrize("N,L,K", [(336, 2, (21, 2)), (100, 1, 7), (1000, 2, (63, 4))])
@pytest.mark.parametrize("enrich", [False, True])
def test_all_blocks_equal_dense_attention(N, L, K, enrich):
    """Every existing block selected at every level: without enrichment the
    result is dense attention over the N tokens; with it, dense attention over
    the tokens followed by every level's slice means (the pooled tokens)."""
    G, d = 1, 8
    q, k, v = (_rand((G, N, d), s) for s in (3, 4, 5))
    s = 1.0 / np.sqrt(d)
    r = oracle.run(q, k, v, BS, L, K, flags=0 if enrich else oracle.NO_ENRICH)
    keys, vals = [k], [v]
    if enrich:
        for l in range(1, L + 1):
            keys.append(_slice_means(k, BS ** l))
            vals.append(_slice_means(v, BS ** l))
    o, lse = _dense(q, np.concatenate(keys, 1), np.concatenate(vals, 1), s)
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


def test_padded_dense_gradient_closed_form():
    """All blocks, no enrichment, N = 336: the gradient of dense attention."""
    G, N, d, L, K = 1, 336, 8, 2, (21, 2)
    q, k, v, do = (_rand((G, N, d), s) for s in (6, 7, 8, 9))
    s = 1.0 / np.sqrt(d)
    r = oracle.run(q, k, v, BS, L, K, flags=oracle.NO_ENRICH, dout=do)
    z = s * q @ k.transpose(0, 2, 1)
    P = np.exp(z - z.max(2, keepdims=True))
    P /= P.sum(2, keepdims=True)
    o = P @ v
    dS = P * (do @ v.transpose(0, 2, 1) - (do * o).sum(2, keepdims=True))
    np.testing.assert_allclose(r["dv"], P.transpose(0, 2, 1) @ do, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dq"], s * dS @ k, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dk"], s * dS.transpose(0, 2, 1) @ q, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,L,K,flags", [(336, 2, (4, 2), 0), (336, 2, (4, 2), oracle.SIZE_BIAS),
                                         (100, 1, 3, 0), (1000, 2, (3, 2), 0)])
def test_padded_finite_differences(N, L, K, flags):
    """Central differences of <dO, O> with the selection held fixed, on
    coordinates that include every token of the partial last blocks (their
    pooled tokens average fewer than 16^l tokens)."""
    G, d = 1, 8
    rng = np.random.default_rng(N + flags)
    q, k, v, do = (rng.standard_normal((G, N, d)) for _ in range(4))
    r = oracle.run(q, k, v, BS, L, K, flags=flags, dout=do)
    grads = {"q": r["dq"], "k": r["dk"], "v": r["dv"]}
    span = BS ** L
    tail = range((N - 1) // span * span, N)  # tokens of the last (partial) top block
    eps = 1e-6
    checked = skipped = total = 0
    for name in ("q", "k", "v"):
        coords = [(0, int(t), int(c)) for t, c in zip(rng.integers(0, N, 30),
                                                       rng.integers(0, d, 30))]
        coords += [(0, t, (t * 5) % d) for t in list(tail)[:: max(1, len(tail) // 20)]]
        total += len(coords)
        for co in coords:
            vals, flipped = [], False
            for sgn in (1, -1):
                args = {"q": q, "k": k, "v": v}
                x = args[name].copy()
                x[co] += sgn * eps
                args[name] = x
                rr = oracle.run(args["q"], args["k"], args["v"], BS, L, K, flags=flags)
                flipped |= any(not np.array_equal(a, b) for a, b in zip(rr["idx"], r["idx"]))
                vals.append(float((rr["out"] * do).sum()))
            if flipped:
                skipped += 1
                continue
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grads[name][co]) <= 1e-6 * max(1.0, abs(fd)), (name, co, fd,
                                                                          grads[name][co])
            checked += 1
    assert checked >= 0.9 * total
