/*
 * llsa_oracle.h -- plain, slow, fp64 CPU oracle for Log-linear Sparse
 * Attention (LLSA).  TEST INFRASTRUCTURE ONLY: used by the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark, never by the product
 * path.  It shares no code with the HIP library.
 *
 * Sources (the method, as described on the pages):
 *   [P1] LLSA GitHub README: usage (drop-in replacement of non-causal
 *        scaled-dot-product attention, block_size=16, power-of-two token
 *        count and top-k), and the quadtree token reordering for images.
 *   [P2] "Log Linear Sparse Attention" skill summary, "Core Technique":
 *        (1) hierarchical compression with Top-K selection that, below the
 *        coarsest level, only scores the children of the indices found at the
 *        level above; (2) hierarchical KV enrichment with coarse tokens from
 *        several levels; (3) a sparse index transpose for the backward pass
 *        instead of a dense mask.
 *   [P3] arXiv 2512.16615 abstract: block-wise compression of tokens and
 *        Top-K selection of key blocks.
 *
 * Conventions (all arrays contiguous, row-major):
 *   G = B*H independent heads, N tokens, d channels, bs = block size,
 *   L = number of pooling levels, K[l-1] = top-k of level l (all equal in the
 *   README's usage; a per-level K is an extension),
 *   n_l = ceil(N / bs^l) blocks at level l (l = 1..L): block j covers tokens
 *   j*bs^l .. min((j+1)*bs^l, N) - 1, so when bs^l does not divide N the last
 *   block of a level is partial (padding to a multiple of bs^L, with the
 *   padded tokens never attended).
 *   token tensors  : [G][N][d]            double
 *   pyramid        : level l (1..L) stored at offset G*d*sum_{l'<l} n_{l'},
 *                    each level [G][n_l][d]
 *   index pyramid  : level l stored at offset G*sum_{l'<l} n_{l'}*K[l'-1],
 *                    each level [G][n_l][K[l-1]], ascending within a row
 *   gap pyramid    : level l at offset G*sum_{l'<l} n_{l'}, each [G][n_l]
 *   lse            : [G][N], natural logarithm
 *
 * Parity pins: every function is checked by tests against values fixed by
 * the pages or by mathematics (closed forms, brute force on tiny inputs,
 * dense-attention special cases, finite differences).
 */
#ifndef LLSA_ORACLE_H
#define LLSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* enrichment variants (flags) */
#define ORC_NO_ENRICH 1u     /* fine tokens only */
#define ORC_ENRICH_COARSE 2u /* pooled tokens of levels 2..L only */
#define ORC_SIZE_BIAS 4u     /* a level-l pooled logit gets + ln bs^l */
#define ORC_ENRICH_COMPLEMENT 8u /* the pooled tokens of the candidates a level did
                                    NOT pick, instead of those it picked */
#define ORC_CAUSAL 16u       /* token t attends keys u <= t (selection: see
                                orc_select_level; not with the complement) */

/* Morton (Z-order) position of raster cell (y, x) on a side x side grid,
 * side a power of two: bits of y and x interleaved, the y bit above the x
 * bit at each scale ([P1], quadtree reordering). */
int64_t orc_morton(int64_t side, int64_t y, int64_t x);

/* Gather src [outer][side*side][inner] (raster order) into dst in Z-order:
 * dst[o][morton(r)][:] = src[o][r][:].  inverse != 0 undoes it. */
void orc_zorder(const double* src, double* dst, int64_t outer, int64_t side,
                int64_t inner, int inverse);

/* Grid order of T frames of H x W cells (T = 1: an image): tiles of the
 * largest power-of-two square (cube when T > 1) dividing every side, in raster
 * order; Morton order inside a tile, frame bit above row bit above column bit
 * ([P1], quadtree reordering, extended to rectangles and video).  Returns the
 * position of cell (t, y, x); for a square power-of-two image it equals
 * orc_morton. */
int64_t orc_grid_index(int64_t T, int64_t H, int64_t W, int64_t t, int64_t y, int64_t x);

/* Gather src [outer][T*H*W][inner] (raster order) into dst in grid order;
 * inverse != 0 undoes it. */
void orc_grid_order(const double* src, double* dst, int64_t outer, int64_t T, int64_t H,
                    int64_t W, int64_t inner, int inverse);

/* Block mean-pool pyramid of x [G][N][d]: level l token i is the mean of the
 * tokens block i covers, computed from its (up to bs) level-(l-1) children
 * weighted by the tokens each covers ([P2] hierarchical compression, [P3]
 * block-wise representation). */
void orc_pool(const double* x, int64_t G, int64_t N, int64_t d, int64_t bs,
              int L, double* pyr);

/* Top-K selection at one level ([P2] hierarchical Top-K).
 * parent == NULL: coarsest level, candidates are all n_l blocks.
 * otherwise parent is [G][ceil(n_l/bs)][Kp] (ascending) and the candidates of
 * row i are the existing children bs*c + r < n_l of the parent row i/bs.
 * Precondition: every row has at least K candidates.
 * Score = scale * <qbar_l[i], kbar_l[j]>; order = score descending, then
 * block index ascending; the first K are kept and stored ascending.
 * gap[i] = score of K-th kept - score of best rejected (+inf if none).
 * causal != 0: the candidates are the blocks j < i among those above (parent
 * entries -1 are unused slots); row i keeps itself and the best K-1 of them
 * (all if fewer), ascending, then -1 in the slots left; gap is that of the
 * K-1 earlier picks. */
void orc_select_level(const double* qbar, const double* kbar,
                      const int32_t* parent, int64_t G, int64_t n_l, int64_t d,
                      int64_t bs, int64_t K, int64_t Kp, double scale, int causal,
                      int32_t* idx, double* gap);

/* All levels, coarsest first (idx, gap in pyramid layouts); K[l-1] picks at
 * level l. */
void orc_select(const double* qpyr, const double* kpyr, int64_t G, int64_t N,
                int64_t d, int64_t bs, int L, const int64_t* K, double scale, int causal,
                int32_t* idx, double* gap);

/* Sparse attention forward with hierarchical KV enrichment.
 * For token t with query block i = t/bs and level-l ancestor a_l = t/bs^l the
 * key/value set is the bs*K[0] tokens of the blocks idx_1[i] plus (unless
 * ORC_NO_ENRICH) the pooled pairs (kbar_l[j], vbar_l[j]) for l = 1..L and
 * j in idx_l[a_l] -- or, with ORC_ENRICH_COMPLEMENT, for j among the
 * candidates of a_l that it did not pick (every level-L block; below L the
 * existing children of the parent's picks).  The fine tokens and the
 * complement's pooled tokens then cover every key token exactly once, each
 * pooled token standing for the tokens it averages.  ORC_CAUSAL: of the
 * diagonal block (the query's own) only the keys u <= t, and no pooled token
 * of an ancestor's own block; -1 picks are skipped.  One softmax over that set with the given scale;
 * lse = m + ln(sum exp(z - m)).
 * qblocks: optional list of query blocks to compute (NULL = all of them, in
 * which case nq is ignored); rows not listed are left untouched. */
void orc_forward(const double* q, const double* k, const double* v,
                 const double* kpyr, const double* vpyr, const int32_t* idx,
                 int64_t G, int64_t N, int64_t d, int64_t bs, int L, const int64_t* K,
                 double scale, unsigned flags, const int64_t* qblocks,
                 int64_t nq, double* out, double* lse);

/* Backward of orc_forward given o, lse (from orc_forward) and dO.
 * dq is written for the query blocks in qblocks (NULL = all); dk, dv are
 * written for the key blocks in kblocks (NULL = all); the rest is untouched.
 * Selection is piecewise constant: no gradient flows through the scores.
 * A pooled token passes 1/count of its gradient to each of the count tokens it
 * averages (mean rule). */
void orc_backward(const double* q, const double* k, const double* v,
                  const double* kpyr, const double* vpyr, const int32_t* idx,
                  const double* o, const double* lse, const double* dout,
                  int64_t G, int64_t N, int64_t d, int64_t bs, int L, const int64_t* K,
                  double scale, unsigned flags, const int64_t* qblocks,
                  int64_t nq, const int64_t* kblocks, int64_t nk, double* dq,
                  double* dk, double* dv);

/* Sparse index transpose of one level ([P2] technique 3): for the index lists
 * idx [G][n][K], col/rowptr hold, per head, T[j] = ascending {i : j in idx[i]}
 * in CSR form: rowptr [G][n+1] (per-head offsets from 0), col [G][n*K];
 * entries -1 (unused slots) are skipped. */
void orc_transpose(const int32_t* idx, int64_t G, int64_t n, int64_t K,
                   int32_t* rowptr, int32_t* col);

#ifdef __cplusplus
}
#endif
#endif
