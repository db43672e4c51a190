"""Pins of the oracle's sparse attention forward with KV enrichment.

LLSA README (page 1, usage): a drop-in replacement of non-causal scaled
dot-product attention, so with every block selected and no enrichment it must
equal dense softmax attention.  Enrichment (page 2, "Core Technique" 2) adds
the pooled tokens of the selected blocks of every level to the key/value set.
"""
import numpy as np
import pytest

import oracle

BS = 16


def dense_attention(q, k, v, scale):
    z = scale * np.einsum("gtc,guc->gtu", q, k)
    m = z.max(axis=2, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=2, keepdims=True)
    return np.einsum("gtu,guc->gtc", p / l, v), (m + np.log(l))[..., 0]


def dense_mask_reference(q, k, v, idx, scale, enrich=True):
    """Independent formulation: one masked softmax per token over all fine
    tokens plus all pooled tokens of every level, the mask built densely from
    the index lists."""
    G, N, d = q.shape
    L = len(idx)
    n1 = N // BS
    out = np.zeros_like(q)
    lse = np.zeros((G, N))
    for g in range(G):
        cols_k = [k[g]]
        cols_v = [v[g]]
        for l in range(1, L + 1):
            cols_k.append(k[g].reshape(N // BS ** l, BS ** l, d).mean(axis=1))
            cols_v.append(v[g].reshape(N // BS ** l, BS ** l, d).mean(axis=1))
        Kc, Vc = np.concatenate(cols_k), np.concatenate(cols_v)
        mask = np.zeros((N, Kc.shape[0]), bool)
        for t in range(N):
            i = t // BS
            blk = np.zeros(n1, bool)
            blk[idx[0][g, i]] = True
            mask[t, :N] = np.repeat(blk, BS)
            if enrich:
                off = N
                for l in range(1, L + 1):
                    n = N // BS ** l
                    mask[t, off + idx[l - 1][g, t // BS ** l]] = True
                    off += n
        z = scale * (q[g] @ Kc.T)
        z = np.where(mask, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        s = p.sum(axis=1, keepdims=True)
        out[g] = (p / s) @ Vc
        lse[g] = (m + np.log(s))[:, 0]
    return out, lse


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_blocks_no_enrichment_is_dense_attention():
    G, N, d = 2, 512, 16
    q, k, v = (_rand((G, N, d), s) for s in (1, 2, 3))
    n1 = N // BS
    r = oracle.run(q, k, v, BS, 1, n1, flags=oracle.NO_ENRICH)
    o, lse = dense_attention(q, k, v, r["scale"])
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


def test_all_blocks_with_enrichment_is_dense_over_concatenation():
    G, N, d = 1, 512, 16
    q, k, v = (_rand((G, N, d), s) for s in (4, 5, 6))
    n1 = N // BS
    r = oracle.run(q, k, v, BS, 1, n1)
    kb = k.reshape(G, n1, BS, d).mean(axis=2)
    vb = v.reshape(G, n1, BS, d).mean(axis=2)
    o, lse = dense_attention(q, np.concatenate([k, kb], 1), np.concatenate([v, vb], 1),
                             r["scale"])
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,L,K", [(1024, 2, 2), (4096, 2, 4), (256, 1, 4)])
@pytest.mark.parametrize("enrich", [True, False])
def test_matches_dense_mask_formulation(N, L, K, enrich):
    G, d = 2, 8
    q, k, v = (_rand((G, N, d), s + N) for s in (7, 8, 9))
    flags = 0 if enrich else oracle.NO_ENRICH
    r = oracle.run(q, k, v, BS, L, K, flags=flags)
    o, lse = dense_mask_reference(q, k, v, r["idx"], r["scale"], enrich)
    np.testing.assert_allclose(r["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)


def test_zero_query_is_uniform_average():
    G, N, d, L, K = 1, 4096, 8, 2, 4
    q = np.zeros((G, N, d))
    k, v = _rand((G, N, d), 10), _rand((G, N, d), 11)
    r = oracle.run(q, k, v, BS, L, K)
    # Q = 0: blocks 0..K-1 at every level, every logit 0, so the output is the
    # plain average of the 16K fine values and the L*K pooled values.
    n_ent = BS * K + L * K
    np.testing.assert_allclose(r["lse"], np.log(n_ent), rtol=0, atol=1e-13)
    fine = v[0, :BS * K].sum(axis=0)
    pooled = sum(v[0, :BS ** l * K].reshape(K, BS ** l, d).mean(axis=1).sum(axis=0)
                 for l in range(1, L + 1))
    want = (fine + pooled) / n_ent
    np.testing.assert_allclose(r["out"][0], np.broadcast_to(want, (N, d)), rtol=0, atol=1e-13)


def test_constant_values_give_constant_output():
    G, N, d = 2, 1024, 8
    q, k = _rand((G, N, d), 12), _rand((G, N, d), 13)
    c = np.linspace(-1, 2, d)
    v = np.broadcast_to(c, (G, N, d)).copy()
    r = oracle.run(q, k, v, BS, 2, 2)
    np.testing.assert_allclose(r["out"], np.broadcast_to(c, (G, N, d)), rtol=0, atol=1e-13)


def test_query_block_subset_matches_full():
    G, N, d = 1, 1024, 8
    q, k, v = (_rand((G, N, d), s) for s in (14, 15, 16))
    r = oracle.run(q, k, v, BS, 2, 2)
    sub = [0, 5, 63]
    o, lse = oracle.forward(q, k, v, r["kpyr"], r["vpyr"], r["idx"], BS, r["scale"],
                            qblocks=sub)
    for i in sub:
        np.testing.assert_array_equal(o[:, BS * i:BS * (i + 1)], r["out"][:, BS * i:BS * (i + 1)])
        np.testing.assert_array_equal(lse[:, BS * i:BS * (i + 1)],
                                      r["lse"][:, BS * i:BS * (i + 1)])
