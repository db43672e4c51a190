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


def dense_mask_reference(q, k, v, idx, scale, enrich=True, first_level=1, size_bias=False):
    """Independent formulation: one masked softmax per token over all fine
    tokens plus all pooled tokens of every level, the mask built densely from
    the index lists.  first_level = 2: pooled tokens of levels 2..L only;
    size_bias: the logit of a level-l pooled token gets + ln(16^l) (it stands
    for 16^l tokens)."""
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
        bias = np.zeros(Kc.shape[0])
        off = N
        for l in range(1, L + 1):
            n = N // BS ** l
            if size_bias:
                bias[off:off + n] = l * np.log(BS)
            off += n
        for t in range(N):
            i = t // BS
            blk = np.zeros(n1, bool)
            blk[idx[0][g, i]] = True
            mask[t, :N] = np.repeat(blk, BS)
            if enrich:
                off = N
                for l in range(1, L + 1):
                    n = N // BS ** l
                    if l >= first_level:
                        mask[t, off + idx[l - 1][g, t // BS ** l]] = True
                    off += n
        z = scale * (q[g] @ Kc.T) + bias[None, :]
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


VARIANTS = {"enrich": 0, "no_enrich": oracle.NO_ENRICH, "coarse": oracle.ENRICH_COARSE,
            "size_bias": oracle.SIZE_BIAS, "coarse_size_bias": oracle.ENRICH_COARSE | oracle.SIZE_BIAS}


@pytest.mark.parametrize("N,L,K", [(1024, 2, 2), (4096, 2, 4), (256, 1, 4),
                                   (1024, 2, (4, 2)), (4096, 3, (2, 5, 1))])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_matches_dense_mask_formulation(N, L, K, variant):
    G, d = 2, 8
    q, k, v = (_rand((G, N, d), s + N) for s in (7, 8, 9))
    flags = VARIANTS[variant]
    r = oracle.run(q, k, v, BS, L, K, flags=flags)
    o, lse = dense_mask_reference(q, k, v, r["idx"], r["scale"],
                                  enrich=not (flags & oracle.NO_ENRICH),
                                  first_level=2 if flags & oracle.ENRICH_COARSE else 1,
                                  size_bias=bool(flags & oracle.SIZE_BIAS))
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


@pytest.mark.parametrize("coarse", [False, True])
def test_zero_query_size_bias_weights_pooled_tokens_by_their_size(coarse):
    """Q = 0 with size-weighted pooled logits: every fine token has weight 1 and a
    level-l pooled token weight 16^l, so out is the weighted mean in closed form
    and lse = ln(16 K + K sum_l 16^l)."""
    G, N, d, L, K = 1, 4096, 8, 2, 4
    q = np.zeros((G, N, d))
    k, v = _rand((G, N, d), 20), _rand((G, N, d), 21)
    flags = oracle.SIZE_BIAS | (oracle.ENRICH_COARSE if coarse else 0)
    r = oracle.run(q, k, v, BS, L, K, flags=flags)
    levels = range(2 if coarse else 1, L + 1)
    total = BS * K + sum(K * BS ** l for l in levels)
    np.testing.assert_allclose(r["lse"], np.log(total), rtol=0, atol=1e-12)
    fine = v[0, :BS * K].sum(axis=0)
    pooled = sum(BS ** l * v[0, :BS ** l * K].reshape(K, BS ** l, d).mean(axis=1).sum(axis=0)
                 for l in levels)
    want = (fine + pooled) / total
    np.testing.assert_allclose(r["out"][0], np.broadcast_to(want, (N, d)), rtol=0, atol=1e-12)


def test_coarse_enrichment_with_one_level_is_no_enrichment():
    """Levels 2..L only, with L = 1, leaves the fine tokens alone."""
    G, N, d = 2, 512, 8
    q, k, v = (_rand((G, N, d), s) for s in (22, 23, 24))
    a = oracle.run(q, k, v, BS, 1, 4, flags=oracle.ENRICH_COARSE)
    b = oracle.run(q, k, v, BS, 1, 4, flags=oracle.NO_ENRICH)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["lse"], b["lse"])
