/*
 * llsa_oracle.c -- plain fp64 CPU oracle for Log-linear Sparse Attention.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).  Every
 * loop below follows the definition of the step it implements, in the order
 * the method describes it; there is no blocking, fusion or reordering.  The
 * sources are listed in llsa_oracle.h ([P1] LLSA README, [P2] LLSA skill
 * summary "Core Technique", [P3] arXiv 2512.16615 abstract).
 */
#include "llsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int64_t ipow(int64_t b, int e)
{
    int64_t r = 1;
    for (int i = 0; i < e; ++i) r *= b;
    return r;
}

/* Blocks of level l: the sequence of N tokens is covered by ceil(N / bs^l)
 * blocks of bs^l consecutive tokens; when bs^l does not divide N the last
 * block is partial (it covers the tokens that remain). */
static int64_t nblk(int64_t N, int64_t bs, int l)
{
    const int64_t span = ipow(bs, l);
    return (N + span - 1) / span;
}

/* tokens covered by block j of level l */
static int64_t blk_tokens(int64_t N, int64_t bs, int l, int64_t j)
{
    const int64_t span = ipow(bs, l), rest = N - j * span;
    return rest < span ? rest : span;
}

/* offset (in rows of width `w`) of level l (1-based) inside a pyramid */
static int64_t lvl_off(int64_t G, int64_t N, int64_t bs, int l, int64_t w)
{
    int64_t off = 0;
    for (int m = 1; m < l; ++m) off += G * nblk(N, bs, m) * w;
    return off;
}

/* offset of level l (1-based) inside an index pyramid whose level-m rows hold
 * K[m-1] entries */
static int64_t idx_off(int64_t G, int64_t N, int64_t bs, int l, const int64_t* K)
{
    int64_t off = 0;
    for (int m = 1; m < l; ++m) off += G * nblk(N, bs, m) * K[m - 1];
    return off;
}

static double dot(const double* a, const double* b, int64_t d)
{
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* ---------------------------------------------------------------- Z-order */

/* [P1] quadtree reordering: at every scale the four quadrants are visited
 * top-left, top-right, bottom-left, bottom-right, i.e. the row bit ranks above
 * the column bit. */
int64_t orc_morton(int64_t side, int64_t y, int64_t x)
{
    int64_t m = 0, w = 1;
    for (int64_t s = 1; s < side; s <<= 1) {
        int64_t yb = (y & s) ? 1 : 0, xb = (x & s) ? 1 : 0;
        m += (2 * yb + xb) * w;
        w *= 4;
    }
    return m;
}

void orc_zorder(const double* src, double* dst, int64_t outer, int64_t side,
                int64_t inner, int inverse)
{
    int64_t n = side * side;
    for (int64_t o = 0; o < outer; ++o)
        for (int64_t r = 0; r < n; ++r) {
            int64_t z = orc_morton(side, r / side, r % side);
            const double* s = src + (o * n + (inverse ? z : r)) * inner;
            double* t = dst + (o * n + (inverse ? r : z)) * inner;
            memcpy(t, s, (size_t)inner * sizeof(double));
        }
}

/* Grid order for images that are not square powers of two and for video
 * ([P1] reorders images "or videos" by a quadtree; the same rule in three
 * dimensions is an octree).  A grid of T frames of H x W cells is cut into
 * tiles of S x S cells (S x S x S cells when T > 1), S the largest power of
 * two that divides every side; tiles come in raster order (frame, row,
 * column), and inside a tile the cells come in Morton order with, at every
 * scale, the frame bit above the row bit above the column bit.  A square
 * power-of-two image is a single tile, so the order is orc_morton's. */
static int64_t pow2_part(int64_t n) { return n & -n; }

int64_t orc_grid_index(int64_t T, int64_t H, int64_t W, int64_t t, int64_t y, int64_t x)
{
    int64_t S = pow2_part(H) < pow2_part(W) ? pow2_part(H) : pow2_part(W);
    const int video = T > 1;
    if (video && pow2_part(T) < S) S = pow2_part(T);
    const int64_t tile = ((video ? t / S : 0) * (H / S) + y / S) * (W / S) + x / S;
    const int64_t cells = video ? S * S * S : S * S;
    int64_t code = 0, w = 1;
    for (int64_t s = 1; s < S; s <<= 1) {
        const int64_t tb = (t & s) ? 1 : 0, yb = (y & s) ? 1 : 0, xb = (x & s) ? 1 : 0;
        if (video) {
            code += (4 * tb + 2 * yb + xb) * w;
            w *= 8;
        } else {
            code += (2 * yb + xb) * w;
            w *= 4;
        }
    }
    return tile * cells + code;
}

void orc_grid_order(const double* src, double* dst, int64_t outer, int64_t T, int64_t H,
                    int64_t W, int64_t inner, int inverse)
{
    const int64_t n = T * H * W;
    for (int64_t o = 0; o < outer; ++o)
        for (int64_t r = 0; r < n; ++r) {  /* r: raster cell (frame, row, column) */
            const int64_t z = orc_grid_index(T, H, W, r / (H * W), (r / W) % H, r % W);
            const double* s = src + (o * n + (inverse ? z : r)) * inner;
            double* t = dst + (o * n + (inverse ? r : z)) * inner;
            memcpy(t, s, (size_t)inner * sizeof(double));
        }
}

/* ------------------------------------------------------------------ pool */

/* [P2] hierarchical compression: level l = block means of level l-1.  A
 * block's pooled token is the mean of the tokens it covers: each of its (up
 * to bs) children enters with the number of tokens that child covers, so a
 * partial last block averages only its own tokens.  (With every block full
 * the weights are equal powers of bs, and the result is the plain mean of the
 * bs children.) */
void orc_pool(const double* x, int64_t G, int64_t N, int64_t d, int64_t bs,
              int L, double* pyr)
{
    for (int l = 1; l <= L; ++l) {
        int64_t n_prev = l == 1 ? N : nblk(N, bs, l - 1), n_l = nblk(N, bs, l);
        const double* src = (l == 1) ? x : pyr + lvl_off(G, N, bs, l - 1, d);
        double* dst = pyr + lvl_off(G, N, bs, l, d);
        for (int64_t g = 0; g < G; ++g)
            for (int64_t i = 0; i < n_l; ++i)
                for (int64_t c = 0; c < d; ++c) {
                    double s = 0.0, w = 0.0;
                    for (int64_t r = 0; r < bs && bs * i + r < n_prev; ++r) {
                        const double wr = l == 1 ? 1.0 : (double)blk_tokens(N, bs, l - 1, bs * i + r);
                        s += wr * src[(g * n_prev + bs * i + r) * d + c];
                        w += wr;
                    }
                    dst[(g * n_l + i) * d + c] = s / w;
                }
    }
}

/* --------------------------------------------------------------- select */

typedef struct {
    double score;
    int32_t j;
} cand_t;

/* score descending, then block index ascending */
static int cand_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int int_cmp(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x < y) ? -1 : (x > y);
}

void orc_select_level(const double* qbar, const double* kbar,
                      const int32_t* parent, int64_t G, int64_t n_l, int64_t d,
                      int64_t bs, int64_t K, int64_t Kp, double scale, int causal,
                      int32_t* idx, double* gap)
{
    int64_t maxc = parent ? bs * Kp : n_l;
    cand_t* c = (cand_t*)malloc((size_t)maxc * sizeof(cand_t));
    for (int64_t g = 0; g < G; ++g)
        for (int64_t i = 0; i < n_l; ++i) {
            /* candidate blocks of row i (causal: only blocks before it; the
             * block itself is chosen apart, below) */
            int64_t nc = 0;
            if (!parent) {
                for (int64_t j = 0; j < (causal ? i : n_l); ++j) c[nc++].j = (int32_t)j;
            } else {
                /* the children of the parent's picks that exist (the last
                 * parent block may have fewer than bs children) */
                const int32_t* pr = parent + (g * ((n_l + bs - 1) / bs) + i / bs) * Kp;
                for (int64_t p = 0; p < Kp; ++p)
                    for (int64_t r = 0; r < bs; ++r) {
                        const int64_t j = bs * (int64_t)pr[p] + r;
                        if (pr[p] < 0 || j >= n_l || (causal && j >= i)) continue;
                        c[nc++].j = (int32_t)j;
                    }
            }
            if (causal) {
                /* the block itself, then the best K-1 earlier candidates (all
                 * of them if fewer); unused slots hold -1 after the picks */
                for (int64_t e = 0; e < nc; ++e)
                    c[e].score = scale * dot(qbar + (g * n_l + i) * d,
                                             kbar + (g * n_l + c[e].j) * d, d);
                qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
                int32_t* row = idx + (g * n_l + i) * K;
                const int64_t take = nc < K - 1 ? nc : K - 1;
                for (int64_t e = 0; e < take; ++e) row[e] = c[e].j;
                row[take] = (int32_t)i;
                qsort(row, (size_t)(take + 1), sizeof(int32_t), int_cmp);
                for (int64_t e = take + 1; e < K; ++e) row[e] = -1;
                if (gap) gap[g * n_l + i] = nc > K - 1 && K > 1 ? c[K - 2].score - c[K - 1].score
                                                                : INFINITY;
                continue;
            }
            const double* qi = qbar + (g * n_l + i) * d;
            for (int64_t e = 0; e < nc; ++e)
                c[e].score = scale * dot(qi, kbar + (g * n_l + c[e].j) * d, d);
            qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
            /* the callers guarantee nc >= K (a row never has fewer candidates
             * than picks); -1 would mark a missing pick */
            int32_t* row = idx + (g * n_l + i) * K;
            for (int64_t e = 0; e < K; ++e) row[e] = e < nc ? c[e].j : -1;
            qsort(row, (size_t)K, sizeof(int32_t), int_cmp);
            if (gap) gap[g * n_l + i] = (nc > K) ? c[K - 1].score - c[K].score : INFINITY;
        }
    free(c);
}

void orc_select(const double* qpyr, const double* kpyr, int64_t G, int64_t N,
                int64_t d, int64_t bs, int L, const int64_t* K, double scale, int causal,
                int32_t* idx, double* gap)
{
    for (int l = L; l >= 1; --l) {
        int64_t n_l = nblk(N, bs, l);
        const int32_t* parent = (l == L) ? NULL : idx + idx_off(G, N, bs, l + 1, K);
        orc_select_level(qpyr + lvl_off(G, N, bs, l, d), kpyr + lvl_off(G, N, bs, l, d),
                         parent, G, n_l, d, bs, K[l - 1], l == L ? 0 : K[l], scale, causal,
                         idx + idx_off(G, N, bs, l, K),
                         gap ? gap + lvl_off(G, N, bs, l, 1) : NULL);
    }
}

/* ------------------------------------------------------------ KV set */

/* Key/value rows of the set of token t (head g): the bs*K fine tokens of the
 * selected level-1 blocks, then, unless disabled, the pooled pairs of the
 * blocks selected at every level l for the token's level-l ancestor ([P2]
 * hierarchical KV enrichment; with ORC_ENRICH_COARSE only levels 2..L).
 * tag[e] = 0 for a fine entry (ref = token), tag[e] = l for a level-l pooled
 * entry (ref = block). */

/* Additive logit of entry e: with ORC_SIZE_BIAS a level-l pooled token, the
 * mean of bs^l tokens, counts as bs^l copies of itself in the softmax
 * (logit + ln bs^l); otherwise 0. */
static double entry_bias(int tag, int64_t bs, unsigned flags)
{
    return (tag > 0 && (flags & ORC_SIZE_BIAS)) ? (double)tag * log((double)bs) : 0.0;
}

static int64_t kv_set(const double* k, const double* v, const double* kpyr,
                      const double* vpyr, const int32_t* idx, int64_t g,
                      int64_t t, int64_t G, int64_t N, int64_t d, int64_t bs,
                      int L, const int64_t* K, unsigned flags, const double** key,
                      const double** val, int* tag, int64_t* ref)
{
    int64_t ne = 0;
    int64_t n1 = nblk(N, bs, 1);
    const int causal = (flags & ORC_CAUSAL) != 0;
    const int32_t* sel1 = idx + (g * n1 + t / bs) * K[0];
    for (int64_t p = 0; p < K[0]; ++p)
        for (int64_t r = 0; sel1[p] >= 0 && r < bs && bs * sel1[p] + r < N; ++r) {
            int64_t u = bs * sel1[p] + r;
            if (causal && u > t) break;  /* the diagonal block: keys up to t */
            key[ne] = k + (g * N + u) * d;
            val[ne] = v + (g * N + u) * d;
            tag[ne] = 0;
            ref[ne] = u;
            ++ne;
        }
    if (!(flags & ORC_NO_ENRICH))
        for (int l = (flags & ORC_ENRICH_COARSE) ? 2 : 1; l <= L; ++l) {
            int64_t n_l = nblk(N, bs, l), a = t / ipow(bs, l);
            const double* kl = kpyr + lvl_off(G, N, bs, l, d);
            const double* vl = vpyr + lvl_off(G, N, bs, l, d);
            const int32_t* sel = idx + idx_off(G, N, bs, l, K) + (g * n_l + a) * K[l - 1];
            if (!(flags & ORC_ENRICH_COMPLEMENT)) {
                /* the pooled tokens of the blocks the ancestor picked (causal:
                 * not its own block, whose mean holds tokens after t) */
                for (int64_t p = 0; p < K[l - 1]; ++p) {
                    int64_t j = sel[p];
                    if (j < 0 || (causal && j == a)) continue;
                    key[ne] = kl + (g * n_l + j) * d;
                    val[ne] = vl + (g * n_l + j) * d;
                    tag[ne] = l;
                    ref[ne] = j;
                    ++ne;
                }
                continue;
            }
            /* the pooled tokens of the ancestor's candidates that it did not
             * pick: every block at the coarsest level, below it the existing
             * children of the parent's picks; ascending */
            int64_t nc = n_l, Kp = 0;
            const int32_t* par = NULL;
            if (l < L) {
                int64_t n_p = nblk(N, bs, l + 1);
                Kp = K[l];
                par = idx + idx_off(G, N, bs, l + 1, K) + (g * n_p + a / bs) * Kp;
                nc = bs * Kp;
            }
            for (int64_t c = 0; c < nc; ++c) {
                const int64_t j = par ? bs * par[c / bs] + c % bs : c;
                if (j >= n_l) continue;  /* the partial last parent has fewer children */
                int picked = 0;
                for (int64_t p = 0; p < K[l - 1]; ++p) picked |= sel[p] == j;
                if (picked) continue;
                key[ne] = kl + (g * n_l + j) * d;
                val[ne] = vl + (g * n_l + j) * d;
                tag[ne] = l;
                ref[ne] = j;
                ++ne;
            }
        }
    return ne;
}

/* Entries a token's key/value set may hold: the fine tokens, then per level
 * the picks, or with ORC_ENRICH_COMPLEMENT the candidates. */
static int64_t max_entries(int64_t N, int64_t bs, int L, const int64_t* K, unsigned flags)
{
    int64_t m = bs * K[0];
    for (int l = 1; l <= L; ++l)
        m += (flags & ORC_ENRICH_COMPLEMENT) ? (l == L ? nblk(N, bs, l) : bs * K[l]) : K[l - 1];
    return m;
}

/* ------------------------------------------------------------- forward */

void orc_forward(const double* q, const double* k, const double* v,
                 const double* kpyr, const double* vpyr, const int32_t* idx,
                 int64_t G, int64_t N, int64_t d, int64_t bs, int L, const int64_t* K,
                 double scale, unsigned flags, const int64_t* qblocks,
                 int64_t nq, double* out, double* lse)
{
    int64_t n1 = nblk(N, bs, 1), maxe = max_entries(N, bs, L, K, flags);
    const double** key = (const double**)malloc((size_t)maxe * sizeof(double*));
    const double** val = (const double**)malloc((size_t)maxe * sizeof(double*));
    int* tag = (int*)malloc((size_t)maxe * sizeof(int));
    int64_t* ref = (int64_t*)malloc((size_t)maxe * sizeof(int64_t));
    double* z = (double*)malloc((size_t)maxe * sizeof(double));
    int64_t nb = qblocks ? nq : n1;
    for (int64_t g = 0; g < G; ++g)
        for (int64_t b = 0; b < nb; ++b) {
            int64_t i = qblocks ? qblocks[b] : b;
            for (int64_t t = bs * i; t < bs * (i + 1) && t < N; ++t) {
                int64_t ne = kv_set(k, v, kpyr, vpyr, idx, g, t, G, N, d, bs, L, K,
                                    flags, key, val, tag, ref);
                const double* qt = q + (g * N + t) * d;
                double m = -INFINITY;
                for (int64_t e = 0; e < ne; ++e) {
                    z[e] = scale * dot(qt, key[e], d) + entry_bias(tag[e], bs, flags);
                    if (z[e] > m) m = z[e];
                }
                double l = 0.0;
                for (int64_t e = 0; e < ne; ++e) l += exp(z[e] - m);
                double* ot = out + (g * N + t) * d;
                for (int64_t c = 0; c < d; ++c) {
                    double s = 0.0;
                    for (int64_t e = 0; e < ne; ++e) s += exp(z[e] - m) * val[e][c];
                    ot[c] = s / l;
                }
                lse[g * N + t] = m + log(l);
            }
        }
    free(key); free(val); free(tag); free(ref); free(z);
}

/* ------------------------------------------------------------ backward */

void orc_backward(const double* q, const double* k, const double* v,
                  const double* kpyr, const double* vpyr, const int32_t* idx,
                  const double* o, const double* lse, const double* dout,
                  int64_t G, int64_t N, int64_t d, int64_t bs, int L, const int64_t* K,
                  double scale, unsigned flags, const int64_t* qblocks,
                  int64_t nq, const int64_t* kblocks, int64_t nk, double* dq,
                  double* dk, double* dv)
{
    int64_t n1 = nblk(N, bs, 1), maxe = max_entries(N, bs, L, K, flags);
    const double** key = (const double**)malloc((size_t)maxe * sizeof(double*));
    const double** val = (const double**)malloc((size_t)maxe * sizeof(double*));
    int* tag = (int*)malloc((size_t)maxe * sizeof(int));
    int64_t* ref = (int64_t*)malloc((size_t)maxe * sizeof(int64_t));

    /* which query blocks need dq; which key blocks need dk/dv; which pooled
     * blocks (per level) feed a needed key block through the mean */
    char* want_q = (char*)calloc((size_t)n1, 1);
    char* want_k = (char*)calloc((size_t)n1, 1);
    if (qblocks) for (int64_t b = 0; b < nq; ++b) want_q[qblocks[b]] = 1;
    else memset(want_q, 1, (size_t)n1);
    if (kblocks) for (int64_t b = 0; b < nk; ++b) want_k[kblocks[b]] = 1;
    else memset(want_k, 1, (size_t)n1);
    int64_t pyr_rows = lvl_off(1, N, bs, L + 1, 1); /* sum_l n_l */
    char* want_p = (char*)calloc((size_t)pyr_rows, 1);
    for (int l = 1; l <= L; ++l)
        for (int64_t j = 0; j < n1; ++j)
            if (want_k[j]) want_p[lvl_off(1, N, bs, l, 1) + j / ipow(bs, l - 1)] = 1;

    /* gradients of the pooled keys / values of one head */
    double* dkp = (double*)malloc((size_t)(pyr_rows * d) * sizeof(double));
    double* dvp = (double*)malloc((size_t)(pyr_rows * d) * sizeof(double));

    for (int64_t g = 0; g < G; ++g) {
        memset(dkp, 0, (size_t)(pyr_rows * d) * sizeof(double));
        memset(dvp, 0, (size_t)(pyr_rows * d) * sizeof(double));
        for (int64_t b = 0; b < n1; ++b)
            if (want_k[b])
                for (int64_t x = bs * b; x < bs * (b + 1) && x < N; ++x)
                    for (int64_t c = 0; c < d; ++c) {
                        dk[(g * N + x) * d + c] = 0.0;
                        dv[(g * N + x) * d + c] = 0.0;
                    }

        for (int64_t i = 0; i < n1; ++i) {
            /* skip query blocks that contribute to no requested output (all
             * tokens of block i share one key/value set) */
            int need = want_q[i];
            if (!need) {
                int64_t ne = kv_set(k, v, kpyr, vpyr, idx, g, bs * i, G, N, d, bs, L, K, flags,
                                    key, val, tag, ref);
                for (int64_t e = 0; e < ne && !need; ++e)
                    need = tag[e] == 0 ? want_k[ref[e] / bs]
                                       : want_p[lvl_off(1, N, bs, tag[e], 1) + ref[e]];
            }
            if (!need) continue;

            for (int64_t t = bs * i; t < bs * (i + 1) && t < N; ++t) {
                int64_t ne = kv_set(k, v, kpyr, vpyr, idx, g, t, G, N, d, bs, L, K,
                                    flags, key, val, tag, ref);
                const double* qt = q + (g * N + t) * d;
                const double* dot_ = dout + (g * N + t) * d;
                double Dt = dot(dot_, o + (g * N + t) * d, d);
                double lt = lse[g * N + t];
                double* dqt = dq + (g * N + t) * d;
                if (want_q[i])
                    for (int64_t c = 0; c < d; ++c) dqt[c] = 0.0;
                for (int64_t e = 0; e < ne; ++e) {
                    double P = exp(scale * dot(qt, key[e], d) + entry_bias(tag[e], bs, flags) - lt);
                    double dP = dot(dot_, val[e], d);
                    double dS = P * (dP - Dt);
                    if (want_q[i])
                        for (int64_t c = 0; c < d; ++c) dqt[c] += scale * dS * key[e][c];
                    double *gk, *gv;
                    if (tag[e] == 0) {
                        if (!want_k[ref[e] / bs]) continue;
                        gk = dk + (g * N + ref[e]) * d;
                        gv = dv + (g * N + ref[e]) * d;
                    } else {
                        int64_t row = lvl_off(1, N, bs, tag[e], 1) + ref[e];
                        if (!want_p[row]) continue;
                        gk = dkp + row * d;
                        gv = dvp + row * d;
                    }
                    for (int64_t c = 0; c < d; ++c) {
                        gk[c] += scale * dS * qt[c];
                        gv[c] += P * dot_[c];
                    }
                }
            }
        }

        /* a level-l pooled token is the mean of the tokens it covers (bs^l,
         * fewer in a partial last block): each of them receives that fraction
         * of its gradient */
        for (int64_t b = 0; b < n1; ++b)
            if (want_k[b])
                for (int64_t x = bs * b; x < bs * (b + 1) && x < N; ++x)
                    for (int l = 1; l <= L; ++l) {
                        int64_t row = lvl_off(1, N, bs, l, 1) + x / ipow(bs, l);
                        double w = 1.0 / (double)blk_tokens(N, bs, l, x / ipow(bs, l));
                        for (int64_t c = 0; c < d; ++c) {
                            dk[(g * N + x) * d + c] += w * dkp[row * d + c];
                            dv[(g * N + x) * d + c] += w * dvp[row * d + c];
                        }
                    }
    }
    free(key); free(val); free(tag); free(ref);
    free(want_q); free(want_k); free(want_p); free(dkp); free(dvp);
}

/* ----------------------------------------------------------- transpose */

/* [P2] technique 3: the key-block -> query-block lists are read off the
 * query-block -> key-block lists; no dense mask.  Rows are visited in
 * ascending order, so every output list comes out ascending. */
void orc_transpose(const int32_t* idx, int64_t G, int64_t n, int64_t K,
                   int32_t* rowptr, int32_t* col)
{
    int32_t* fill = (int32_t*)malloc((size_t)n * sizeof(int32_t));
    for (int64_t g = 0; g < G; ++g) {
        int32_t* rp = rowptr + g * (n + 1);
        int32_t* cl = col + g * n * K;
        const int32_t* I = idx + g * n * K;
        for (int64_t j = 0; j <= n; ++j) rp[j] = 0;
        for (int64_t e = 0; e < n * K; ++e)
            if (I[e] >= 0) rp[I[e] + 1] += 1;  /* -1: an unused slot */
        for (int64_t j = 0; j < n; ++j) rp[j + 1] += rp[j];
        for (int64_t j = 0; j < n; ++j) fill[j] = 0;
        for (int64_t i = 0; i < n; ++i)
            for (int64_t p = 0; p < K; ++p) {
                int32_t j = I[i * K + p];
                if (j >= 0) cl[rp[j] + fill[j]++] = (int32_t)i;
            }
    }
    free(fill);
}
