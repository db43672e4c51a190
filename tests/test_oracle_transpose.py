"""Pins of the oracle's sparse index transpose.

LLSA skill summary (page 2, "Core Technique" 3): the backward pass turns the
query-block -> key-block lists into key-block -> query-block lists directly
from the sparse indices, without a dense mask.  The result must equal the
transpose of the dense block mask.
"""
import numpy as np
import pytest

import oracle

BS = 16


def dense_mask_transpose(idx):
    G, n, K = idx.shape
    out = []
    for g in range(G):
        mask = np.zeros((n, n), bool)
        mask[np.repeat(np.arange(n), K), idx[g].ravel()] = True
        out.append([np.nonzero(mask[:, j])[0] for j in range(n)])
    return out


@pytest.mark.parametrize("N,L,K", [(1024, 1, 8), (4096, 2, 4), (65536, 2, 16)])
def test_transpose_equals_dense_mask_transpose(N, L, K):
    rng = np.random.default_rng(N + K)
    G, d = 2, 4
    q, k = rng.standard_normal((G, N, d)), rng.standard_normal((G, N, d))
    qp, kp = oracle.pool(q, BS, L), oracle.pool(k, BS, L)
    idx, _ = oracle.select(qp, kp, K, BS, 0.5)
    for lvl in idx:
        G_, n, _ = lvl.shape
        rowptr, col = oracle.transpose(lvl)
        want = dense_mask_transpose(lvl)
        assert rowptr.shape == (G, n + 1) and col.shape == (G, n * K)
        for g in range(G):
            assert rowptr[g, 0] == 0 and rowptr[g, -1] == n * K
            for j in range(n):
                np.testing.assert_array_equal(col[g, rowptr[g, j]:rowptr[g, j + 1]], want[g][j])


def test_transpose_degenerate_all_rows_same():
    # every row selects blocks 0..K-1: those K lists hold every row, the rest
    # are empty
    G, n, K = 1, 256, 4
    idx = np.broadcast_to(np.arange(K, dtype=np.int32), (G, n, K)).copy()
    rowptr, col = oracle.transpose(idx)
    for j in range(n):
        seg = col[0, rowptr[0, j]:rowptr[0, j + 1]]
        np.testing.assert_array_equal(seg, np.arange(n) if j < K else [])
