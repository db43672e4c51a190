"""Pins of the oracle's hierarchical Top-K selection.

LLSA skill summary (page 2, "Core Technique" 1): Top-K over pooled blocks,
dense only at the coarsest level; each finer level only scores the children of
the blocks chosen one level up.  Ties go to the lower block index and each
list is stored ascending (readings of this build; the pages do not fix them).
"""
import numpy as np
import pytest

import oracle

BS = 16


def brute_topk(qbar, kbar, cands, K, scale):
    """Independent brute force: numpy scores + lexsort (score desc, index asc)."""
    s = scale * (kbar[cands] @ qbar)
    order = np.lexsort((cands, -s))
    keep = np.sort(cands[order[:K]])
    gap = s[order[K - 1]] - s[order[K]] if len(cands) > K else np.inf
    return keep, gap


def check_hierarchy(qpyr, kpyr, idx, gap, K, scale):
    """K: one top-k for every level, or one per level (level 1 first)."""
    G = qpyr[0].shape[0]
    L = len(qpyr)
    ks = [K] * L if np.isscalar(K) else list(K)
    for l in range(L, 0, -1):
        n = qpyr[l - 1].shape[1]
        Kl = ks[l - 1]
        assert idx[l - 1].shape == (G, n, Kl)
        for g in range(G):
            for i in range(n):
                if l == L:
                    cands = np.arange(n)
                else:
                    par = idx[l][g, i // BS]
                    cands = (BS * par[:, None] + np.arange(BS)[None, :]).ravel()
                keep, gp = brute_topk(qpyr[l - 1][g, i], kpyr[l - 1][g], cands, Kl, scale)
                np.testing.assert_array_equal(idx[l - 1][g, i], keep)
                if np.isinf(gp):
                    assert np.isinf(gap[l - 1][g, i])
                else:
                    assert abs(gap[l - 1][g, i] - gp) <= 1e-12


@pytest.mark.parametrize("N,L,K", [(256, 1, 4), (1024, 1, 8), (1024, 2, 2), (4096, 2, 4),
                                   (4096, 3, 1),
                                   # a top-k per level (level 1 first)
                                   (1024, 2, (4, 2)), (4096, 2, (3, 8)), (1024, 2, (32, 3)),
                                   (4096, 3, (2, 5, 1)), (65536, 3, (6, 3, 9))])
def test_select_matches_brute_force(N, L, K):
    rng = np.random.default_rng(N + L + int(np.sum(K)))
    G, d = 2, 8
    q, k = rng.standard_normal((G, N, d)), rng.standard_normal((G, N, d))
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    scale = 1 / np.sqrt(d)
    idx, gap = oracle.select(qp, kp, K, BS, scale)
    check_hierarchy(qp, kp, idx, gap, K, scale)


def test_children_invariant():
    rng = np.random.default_rng(5)
    G, N, d, L, K = 1, 65536, 4, 3, 2
    q, k = rng.standard_normal((G, N, d)), rng.standard_normal((G, N, d))
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    idx, _ = oracle.select(qp, kp, K, BS, 0.5)
    for l in range(1, L):
        child, par = idx[l - 1][0], idx[l][0]
        for i in range(child.shape[0]):
            assert set((child[i] // BS).tolist()) <= set(par[i // BS].tolist())
            assert np.all(np.diff(child[i]) > 0)


def test_exact_ties_go_to_lower_index():
    # key blocks 3, 9 and 12 are identical copies of block 5: their scores
    # tie bit-exactly, so with K=2 the winners among them are the two lowest.
    rng = np.random.default_rng(6)
    G, N, d, K = 1, 256, 8, 2
    q = rng.standard_normal((G, N, d))
    k = rng.standard_normal((G, N, d)) * 0.01
    big = rng.standard_normal(d)
    for j in (3, 5, 9, 12):
        k[0, 16 * j:16 * (j + 1)] = big + rng.standard_normal(d)[None, :] * 0  # same rows
    qp, kp = oracle.pool(q, BS, 1), oracle.pool(k, BS, 1)
    # make the query prefer this direction strongly
    qp[0][0, 0] = big * 10
    idx, gap = oracle.select_level(qp[0], kp[0], None, K, BS, 1.0)
    np.testing.assert_array_equal(idx[0, 0], [3, 5])
    assert gap[0, 0] == 0.0


def test_zero_query_selects_first_blocks():
    # Q = 0 makes every score exactly 0: the tie rule picks blocks 0..K-1 at the
    # coarsest level and the lowest children at every finer level.
    rng = np.random.default_rng(7)
    G, N, d, L, K = 2, 4096, 8, 2, 4
    q = np.zeros((G, N, d))
    k = rng.standard_normal((G, N, d))
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    idx, _ = oracle.select(qp, kp, K, BS, 0.125)
    for lvl in idx:
        assert np.all(lvl == np.arange(K)[None, None, :])


def test_two_levels_with_all_parents_equals_one_level():
    # K = n_2 keeps every level-2 block, so the level-1 candidates are all
    # blocks and the level-1 choice must equal the single-level choice.
    rng = np.random.default_rng(8)
    G, N, d = 2, 1024, 8
    K = N // 256
    q, k = rng.standard_normal((G, N, d)), rng.standard_normal((G, N, d))
    qp, kp = oracle.pool(q, BS, 2), oracle.pool(k, BS, 2)
    idx2, _ = oracle.select(qp, kp, K, BS, 0.3)
    idx1, _ = oracle.select(qp[:1], kp[:1], K, BS, 0.3)
    np.testing.assert_array_equal(idx2[0], idx1[0])


def test_planted_block_selected_at_every_level():
    rng = np.random.default_rng(9)
    G, N, d, L, K = 1, 4096, 16, 2, 2
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((G, N, d))
    k = rng.standard_normal((G, N, d))
    q[0, :256] = u  # level-2 query block 0 (and its 16 children) points along u
    jstar = 16 * 7 + 3  # key block 115, inside level-2 block 7
    k[0, 16 * jstar:16 * (jstar + 1)] = 200.0 * u
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    idx, _ = oracle.select(qp, kp, K, BS, 0.25)
    assert 7 in idx[1][0, 0]
    for i in range(16):
        assert jstar in idx[0][0, i]
