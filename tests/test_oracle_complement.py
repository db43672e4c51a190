"""Pins of the complement enrichment variant (ORC_ENRICH_COMPLEMENT).

The skill summary (page 2, "Core Technique" 2) enriches the key/value set
with coarse tokens from several levels to preserve global context with fewer
tokens, without saying which ones.  Reading R2b: at every level the pooled
tokens of the candidates the query's ancestor did NOT pick (every block at the
coarsest level; below it the existing children of the parent's picks).  The
fine tokens and those pooled tokens then cover every key token exactly once,
each pooled token standing for the tokens it averages.

Pins: a closed form (Q = 0 with size-weighted logits gives, for every query,
the mean of all N values and lse = ln N -- it holds only because the cover is
a partition); an independent numpy construction of each query's set;
every block selected (the complement is empty: dense attention); finite
differences of the backward.
"""
import numpy as np
import pytest

import oracle

BS = 16
CMP = oracle.ENRICH_COMPLEMENT


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N,L,K", [(256, 1, 4), (1024, 2, 2), (1024, 2, (3, 2)),
                                   (16384, 3, (2, 3, 2)), (4096, 2, (8, 4))])
def test_zero_queries_with_size_bias_average_every_token(N, L, K):
    G, d = 2, 8
    q = np.zeros((G, N, d))
    k, v = _rand((G, N, d), 1), _rand((G, N, d), 2)
    r = oracle.run(q, k, v, BS, L, K, flags=CMP | oracle.SIZE_BIAS)
    want = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    np.testing.assert_allclose(r["out"], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], np.log(N), rtol=0, atol=1e-12)


def _slice_means(x, span):
    G, N, d = x.shape
    n = -(-N // span)
    return np.stack([x[:, j * span:min((j + 1) * span, N)].mean(axis=1) for j in range(n)], 1)


def _numpy_forward(q, k, v, idx, L, s, size_bias):
    """Each query's key/value set built from its definition, then softmax."""
    G, N, d = q.shape
    n = oracle.level_sizes(N, BS, L)
    kb = [_slice_means(k, BS ** l) for l in range(1, L + 1)]
    vb = [_slice_means(v, BS ** l) for l in range(1, L + 1)]
    out, lse = np.zeros_like(q), np.zeros((G, N))
    for g in range(G):
        for t in range(N):
            keys, vals, bias = [], [], []
            for j in idx[0][g, t // BS]:
                for u in range(BS * j, min(BS * j + BS, N)):
                    keys.append(k[g, u]); vals.append(v[g, u]); bias.append(0.0)
            for l in range(1, L + 1):
                a = t // BS ** l
                picks = set(idx[l - 1][g, a].tolist())
                if l == L:
                    cands = range(n[l - 1])
                else:
                    cands = [BS * c + r for c in idx[l][g, a // BS] for r in range(BS)
                             if BS * c + r < n[l - 1]]
                for j in cands:
                    if j not in picks:
                        keys.append(kb[l - 1][g, j]); vals.append(vb[l - 1][g, j])
                        bias.append(l * np.log(BS) if size_bias else 0.0)
            z = s * np.array(keys) @ q[g, t] + np.array(bias)
            m = z.max()
            p = np.exp(z - m)
            out[g, t] = p @ np.array(vals) / p.sum()
            lse[g, t] = m + np.log(p.sum())
    return out, lse


@pytest.mark.parametrize("N,L,K", [(256, 1, 4), (1024, 2, (3, 2)), (336, 2, (4, 2))])
@pytest.mark.parametrize("size_bias", [False, True])
def test_matches_an_independent_construction(N, L, K, size_bias):
    G, d = 1, 8
    q, k, v = (_rand((G, N, d), s) for s in (3, 4, 5))
    flags = CMP | (oracle.SIZE_BIAS if size_bias else 0)
    r = oracle.run(q, k, v, BS, L, K, flags=flags)
    o, lse = _numpy_forward(q, k, v, r["idx"], L, 1.0 / np.sqrt(d), size_bias)
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


def test_every_block_selected_leaves_no_complement():
    G, N, d = 1, 1024, 8
    q, k, v = (_rand((G, N, d), s) for s in (6, 7, 8))
    r = oracle.run(q, k, v, BS, 2, (64, 4), flags=CMP)  # every level-1 and level-2 block
    z = q @ k.transpose(0, 2, 1) / np.sqrt(d)
    p = np.exp(z - z.max(2, keepdims=True))
    np.testing.assert_allclose(r["out"], (p / p.sum(2, keepdims=True)) @ v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,L,K,flags", [(256, 1, 4, CMP), (1024, 2, 2, CMP),
                                         (1024, 2, (3, 2), CMP | oracle.SIZE_BIAS),
                                         (336, 2, (4, 2), CMP),
                                         (1024, 2, 2, CMP | oracle.ENRICH_COARSE)])
def test_finite_differences(N, L, K, flags):
    G, d = 1, 8
    rng = np.random.default_rng(N + flags)
    q, k, v, do = (rng.standard_normal((G, N, d)) for _ in range(4))
    r = oracle.run(q, k, v, BS, L, K, flags=flags, dout=do)
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
                rr = oracle.run(args["q"], args["k"], args["v"], BS, L, K, flags=flags)
                flipped |= any(not np.array_equal(a, b) for a, b in zip(rr["idx"], r["idx"]))
                vals.append(float((rr["out"] * do).sum()))
            if flipped:
                continue
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grads[name][co]) <= 1e-6 * max(1.0, abs(fd)), (name, co, fd,
                                                                          grads[name][co])
            checked += 1
    assert checked >= 0.9 * total
