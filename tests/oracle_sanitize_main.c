/* Exercises every routine of the CPU oracle on small random inputs, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure: tests/test_oracle_sanitize.py compiles and runs it).  Any
 * out-of-bounds access, leak or undefined operation aborts the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "llsa_oracle.h"

static double urand(unsigned* s)
{
    *s = *s * 1664525u + 1013904223u;
    return ((*s >> 8) & 0xFFFFFF) / (double)0x1000000 - 0.5;
}

static double* rnd(size_t n, unsigned* s)
{
    double* x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = urand(s);
    return x;
}

int main(void)
{
    unsigned s = 12345u;
    const int64_t G = 2, N0 = 1024, d = 8, bs = 16;
    /* grid orders */
    double* img = rnd(G * N0 * 3, &s);
    double* zo = malloc(G * N0 * 3 * sizeof(double));
    double* back = malloc(G * N0 * 3 * sizeof(double));
    orc_zorder(img, zo, G, 32, 3, 0);
    orc_zorder(zo, back, G, 32, 3, 1);
    orc_grid_order(img, zo, G, 4, 16, 16, 3, 0);
    orc_grid_order(zo, back, G, 4, 16, 16, 3, 1);
    orc_grid_order(img, zo, G, 1, 24, 32, 3, 0);
    free(img); free(zo); free(back);

    for (int pad = 0; pad < 2; ++pad)
    for (int L = 1; L <= 2; ++L) {
        /* pad: 336 tokens, partial last blocks (21 level-1 blocks, the second
         * level-2 block covering 5 of them) */
        const int64_t N = pad ? 336 : N0;
        const int64_t Ks[3][2] = {{2, 2}, {3, 2}, {4, 1}};
        for (int kc = 0; kc < 3; ++kc) {
            int64_t K[2] = {Ks[kc][0], Ks[kc][1]};
            if (L == 2 && K[1] > (N + bs * bs - 1) / (bs * bs)) continue;
            double* q = rnd(G * N * d, &s);
            double* k = rnd(G * N * d, &s);
            double* v = rnd(G * N * d, &s);
            double* dout = rnd(G * N * d, &s);
            int64_t rows = 0, irows = 0;
            for (int l = 1; l <= L; ++l) {
                int64_t nl = N;
                for (int m = 0; m < l; ++m) nl = (nl + bs - 1) / bs;
                rows += nl;
                irows += nl * K[l - 1];
            }
            double* qp = malloc(G * rows * d * sizeof(double));
            double* kp = malloc(G * rows * d * sizeof(double));
            double* vp = malloc(G * rows * d * sizeof(double));
            orc_pool(q, G, N, d, bs, L, qp);
            orc_pool(k, G, N, d, bs, L, kp);
            orc_pool(v, G, N, d, bs, L, vp);
            int32_t* idx = malloc(G * irows * sizeof(int32_t));
            double* gap = malloc(G * rows * sizeof(double));
            orc_select(qp, kp, G, N, d, bs, L, K, 1.0 / sqrt((double)d), 0, idx, gap);
            double* o = malloc(G * N * d * sizeof(double));
            double* lse = malloc(G * N * sizeof(double));
            double* dq = malloc(G * N * d * sizeof(double));
            double* dk = malloc(G * N * d * sizeof(double));
            double* dv = malloc(G * N * d * sizeof(double));
            /* a causal selection too (rows with fewer picks hold -1) */
            int32_t* cidx = malloc(G * irows * sizeof(int32_t));
            orc_select(qp, kp, G, N, d, bs, L, K, 1.0 / sqrt((double)d), 1, cidx, gap);
            orc_forward(q, k, v, kp, vp, cidx, G, N, d, bs, L, K, 0.3, 16u, NULL, 0, o, lse);
            orc_backward(q, k, v, kp, vp, cidx, o, lse, dout, G, N, d, bs, L, K, 0.3, 16u,
                         NULL, 0, NULL, 0, dq, dk, dv);
            {
                const int64_t n1c = (N + bs - 1) / bs;
                int32_t* rpc = malloc(G * (n1c + 1) * sizeof(int32_t));
                int32_t* colc = malloc(G * n1c * K[0] * sizeof(int32_t));
                orc_transpose(cidx, G, n1c, K[0], rpc, colc);
                free(rpc); free(colc);
            }
            free(cidx);
            for (unsigned flags = 0; flags < 16; ++flags) {
                orc_forward(q, k, v, kp, vp, idx, G, N, d, bs, L, K, 0.3, flags, NULL, 0, o, lse);
                orc_backward(q, k, v, kp, vp, idx, o, lse, dout, G, N, d, bs, L, K, 0.3, flags,
                             NULL, 0, NULL, 0, dq, dk, dv);
                const int64_t qb[2] = {0, (N + bs - 1) / bs - 1}, kb[1] = {3};
                orc_forward(q, k, v, kp, vp, idx, G, N, d, bs, L, K, 0.3, flags, qb, 2, o, lse);
                orc_backward(q, k, v, kp, vp, idx, o, lse, dout, G, N, d, bs, L, K, 0.3, flags,
                             qb, 2, kb, 1, dq, dk, dv);
            }
            const int64_t n1 = (N + bs - 1) / bs;
            int32_t* rp = malloc(G * (n1 + 1) * sizeof(int32_t));
            int32_t* col = malloc(G * n1 * K[0] * sizeof(int32_t));
            orc_transpose(idx, G, n1, K[0], rp, col);
            double* lvl = malloc(G * n1 * sizeof(double));
            orc_select_level(qp, kp, NULL, G, n1, d, bs, K[0], 0, 0.3, 0, idx, lvl);
            free(q); free(k); free(v); free(dout); free(qp); free(kp); free(vp); free(idx);
            free(gap); free(o); free(lse); free(dq); free(dk); free(dv); free(rp); free(col);
            free(lvl);
        }
    }
    puts("oracle sanitize run ok");
    return 0;
}
