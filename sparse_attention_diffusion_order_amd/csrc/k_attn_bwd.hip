// k_attn_bwd.hip -- backward of the sparse attention with KV enrichment.
//
// LLSA skill summary: the method is trainable and its sparse kernels run in
// both passes; "Core Technique" 3: the key-side gradients are organised by the
// key-block -> query-block lists from the sparse index transpose.
//
// With P = exp(z - lse), D_t = <dO_t, O_t>, dS = P (dP - D), dP = <dO_t, v>:
//   dq_t   = s * sum_e dS_te key_e                (query-major, dq kernels)
//   dk_x   = s * sum_t dS_tx q_t, dv_x = sum_t P_tx dO_t   (key-major over T_1)
//   pooled entry (l, j): same sums into dkbar_l[j], dvbar_l[j], which pass
//   1/16^l of themselves to each of the 16^l tokens they average.
// Selection is piecewise constant: no gradient flows into the scores.
//
// bf16 path:
//   dq_bf16     one wave per query block; S^T = K Q^T and dP^T = V dO^T on
//               MFMA, dQ^T += K^T dS^T with K^T read transposed from LDS;
//               level-1 pooled tokens folded into the tiles exactly as in the
//               forward; also writes D.
//   enrich_bwd  one workgroup per level-2 block (256 query tokens): for each
//               level >= 2 entry list (shared by all 256 tokens) the partial
//               sums over the group, reduced across waves in fixed order.
//   enrich_sum  per pooled block: sum of the partials of the query groups
//               that chose it (found through that level's transpose).
//   dkdv_bf16   one wave per key block over its list T_1[j] (pairs of query
//               blocks form the 32-deep contraction); Q^T and dO^T read
//               transposed from LDS; level-1 pooled token folded in; the
//               epilogue adds the pooled-level gradients.
// fp32 path: plain VALU kernels with explicit pooled tokens at every level.
// No floating-point atomics anywhere: results are bit-identical run to run.
#include "common.h"

namespace llsa {
namespace {

constexpr int LDS_ROW = 80;  // bf16 per staged row (160 B)
constexpr int TILE = BS * LDS_ROW;

__device__ __forceinline__ bf16x8 ld8(const unsigned short* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ bf16x8 ld8f(const float* p)
{
    float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    bf16x8 r;
    r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
    r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
    return r;
}

// Sum over the 16 lanes of a DPP row (lanes 16g .. 16g+15).
__device__ __forceinline__ float row16_sum(float x)
{
    int v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));  // xor 1
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));  // xor 2
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // half mirror
    v = __float_as_int(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // mirror
    return x;
}

__device__ __forceinline__ long enrich_row(const Geo& g, const Ws& w, int gh, int i, int e,
                                           int* level)
{
    int l = 2 + e / g.K, s = e % g.K;
    int a = i >> (4 * (l - 1));
    int j = w.idx[l - 1][((long)gh * g.n[l] + a) * g.K + s];
    *level = l;
    return ((long)gh * g.n[l] + j) * D;
}

// dq tile: key rows staged row-major in LDS (for the transposed K^T read),
// A operands of S^T (key rows) and dP^T (value rows) in registers.
__device__ __forceinline__ int dq_tile(const Geo& g, const Ws& w, const unsigned short* k,
                                       const unsigned short* v, int gh, int i, int t,
                                       int ntiles, unsigned short* lds, bf16x8& k0, bf16x8& k1,
                                       bf16x8& v0, bf16x8& v1, int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    if (t < g.K) {
        int j = w.idx[0][((long)gh * g.n[1] + i) * g.K + t];
        long base = ((long)gh * g.N + (long)j * BS) * D;
        k0 = ld8(k + base + nq * D + 8 * gq);
        k1 = ld8(k + base + nq * D + 32 + 8 * gq);
        v0 = ld8(v + base + nq * D + 8 * gq);
        v1 = ld8(v + base + nq * D + 32 + 8 * gq);
        *(bf16x8*)(lds + sr * LDS_ROW + sc) = ld8(k + base + sr * D + sc);
        *(bf16x8*)(lds + (sr + 8) * LDS_ROW + sc) = ld8(k + base + (sr + 8) * D + sc);
        return BS;
    }
    const int E = (t < ntiles && !(g.flags & LLSA_NO_ENRICH)) ? (g.L - 1) * g.K : 0;
    const int e0 = (t - g.K) * BS;
    const int nvalid = max(0, min(BS, E - e0));
    const bf16x8 z = {};
    k0 = k1 = v0 = v1 = z;
    if (nq < nvalid) {
        int lv;
        long off = enrich_row(g, w, gh, i, e0 + nq, &lv);
        k0 = ld8f(w.kbar[lv - 1] + off + 8 * gq);
        k1 = ld8f(w.kbar[lv - 1] + off + 32 + 8 * gq);
        v0 = ld8f(w.vbar[lv - 1] + off + 8 * gq);
        v1 = ld8f(w.vbar[lv - 1] + off + 32 + 8 * gq);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int row = sr + 8 * h;
        bf16x8 val = z;
        if (row < nvalid) {
            int lv;
            long off = enrich_row(g, w, gh, i, e0 + row, &lv);
            val = ld8f(w.kbar[lv - 1] + off + sc);
        }
        *(bf16x8*)(lds + row * LDS_ROW + sc) = val;
    }
    return nvalid;
}

__global__ __launch_bounds__(256) void dq_bf16(const unsigned short* __restrict__ q,
                                               const unsigned short* __restrict__ k,
                                               const unsigned short* __restrict__ v,
                                               const unsigned short* __restrict__ o,
                                               const float* __restrict__ lse,
                                               const unsigned short* __restrict__ dout,
                                               unsigned short* __restrict__ dq, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][2][TILE];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)blockIdx.x * 4 + wv;
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const bool enrich = !(g.flags & LLSA_NO_ENRICH);
    const float c = g.scale * LOG2E;
    const long qbase = ((long)gh * g.N + (long)i * BS) * D;
    const long rowq = qbase + nq * D;
    const bf16x8 bq0 = ld8(q + rowq + 8 * gq), bq1 = ld8(q + rowq + 32 + 8 * gq);
    const bf16x8 bd0 = ld8(dout + rowq + 8 * gq), bd1 = ld8(dout + rowq + 32 + 8 * gq);
    float Dq;
    {
        const bf16x8 o0 = ld8(o + rowq + 8 * gq), o1 = ld8(o + rowq + 32 + 8 * gq);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += (float)bd0[e] * (float)o0[e] + (float)bd1[e] * (float)o1[e];
        s += shfl_xor(s, 16);
        s += shfl_xor(s, 32);
        Dq = s;
    }
    const long tok = (long)gh * g.N + (long)i * BS + nq;
    if (gq == 0) w.delta[tok] = Dq;
    const float l2 = lse[tok] * LOG2E;

    const int ntiles = g.K + (enrich ? ((g.L - 1) * g.K + BS - 1) / BS : 0);
    f32x4 acc[4] = {};
    unsigned short* la = smem[wv][0];
    unsigned short* lb = smem[wv][1];
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 zero = {};
    for (int ta = 0; ta < ntiles; ta += 2) {
        const int tb = ta + 1;
        bf16x8 ka0, ka1, va0, va1, kb0, kb1, vb0, vb1;
        int na = dq_tile(g, w, k, v, gh, i, ta, ntiles, la, ka0, ka1, va0, va1, lane);
        int nb = dq_tile(g, w, k, v, gh, i, tb, ntiles, lb, kb0, kb1, vb0, vb1, lane);
        f32x4 sa = mfma32(ka1, bq1, mfma32(ka0, bq0, zero));
        f32x4 sb = mfma32(kb1, bq1, mfma32(kb0, bq0, zero));
        f32x4 pa = mfma32(va1, bd1, mfma32(va0, bd0, zero));  // dP^T
        f32x4 pb = mfma32(vb1, bd1, mfma32(vb0, bd0, zero));
        float dsa[4], dsb[4], za[4], zb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            za[r] = sa[r] * c;
            zb[r] = sb[r] * c;
            float Pa = (4 * gq + r < na) ? fast_exp2(za[r] - l2) : 0.f;
            float Pb = (4 * gq + r < nb) ? fast_exp2(zb[r] - l2) : 0.f;
            dsa[r] = Pa * (pa[r] - Dq);
            dsb[r] = Pb * (pb[r] - Dq);
        }
        if (enrich) {
            if (ta < g.K) {
                float zs = za[0] + za[1] + za[2] + za[3], ps = pa[0] + pa[1] + pa[2] + pa[3];
                zs += shfl_xor(zs, 16); zs += shfl_xor(zs, 32);
                ps += shfl_xor(ps, 16); ps += shfl_xor(ps, 32);
                float pe = fast_exp2(zs * (1.0f / BS) - l2);
                float dse = pe * (ps * (1.0f / BS) - Dq) * (1.0f / BS);
#pragma unroll
                for (int r = 0; r < 4; ++r) dsa[r] += dse;
            }
            if (tb < g.K) {
                float zs = zb[0] + zb[1] + zb[2] + zb[3], ps = pb[0] + pb[1] + pb[2] + pb[3];
                zs += shfl_xor(zs, 16); zs += shfl_xor(zs, 32);
                ps += shfl_xor(ps, 16); ps += shfl_xor(ps, 32);
                float pe = fast_exp2(zs * (1.0f / BS) - l2);
                float dse = pe * (ps * (1.0f / BS) - Dq) * (1.0f / BS);
#pragma unroll
                for (int r = 0; r < 4; ++r) dsb[r] += dse;
            }
        }
        bf16x8 bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bs[r] = (bf16)dsa[r];
            bs[4 + r] = (bf16)dsb[r];
        }
        wave_lds_sync();
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
            bf16x4 x0 = lds_read_tr(la + off), x1 = lds_read_tr(lb + off);
            bf16x8 ak = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            acc[d] = mfma32(ak, bs, acc[d]);
        }
        wave_lds_sync();
    }
    const long obase = rowq + 4 * gq;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        u16x4 r4;
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[r] = f2bf(acc[d][r] * g.scale);
        *(u16x4*)(dq + obase + 16 * d) = r4;
    }
}

// Stage a 16-token query-side tile (rows of x) into LDS, zeros if !live.
__device__ __forceinline__ void stage_rows(unsigned short* lds, const unsigned short* x, long base,
                                           bool live, int lane)
{
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    const bf16x8 z = {};
    *(bf16x8*)(lds + sr * LDS_ROW + sc) = live ? ld8(x + base + sr * D + sc) : z;
    *(bf16x8*)(lds + (sr + 8) * LDS_ROW + sc) = live ? ld8(x + base + (sr + 8) * D + sc) : z;
}

__global__ __launch_bounds__(256) void enrich_bwd_bf16(const unsigned short* __restrict__ q,
                                                       const float* __restrict__ lse,
                                                       const unsigned short* __restrict__ dout,
                                                       Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][2][TILE];
    __shared__ float red[4][2][4][4][64];  // [wave][dk|dv][dtile][r][lane]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gq = lane >> 4, nq = lane & 15;
    const int gh = blockIdx.x / g.n[2], a2 = blockIdx.x % g.n[2];
    const float c = g.scale * LOG2E;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    unsigned short* lq = smem[wv][0];
    unsigned short* ld = smem[wv][1];
    const f32x4 zero = {};
    for (int l = 2; l <= g.L; ++l) {
        const int al = a2 >> (4 * (l - 2));
        const int* sel = w.idx[l - 1] + ((long)gh * g.n[l] + al) * g.K;
        for (int e0 = 0; e0 < g.K; e0 += BS) {
            const bool ev = e0 + nq < g.K;
            bf16x8 bk0 = {}, bk1 = {}, bv0 = {}, bv1 = {};
            if (ev) {
                long off = ((long)gh * g.n[l] + sel[e0 + nq]) * D;
                bk0 = ld8f(w.kbar[l - 1] + off + 8 * gq);
                bk1 = ld8f(w.kbar[l - 1] + off + 32 + 8 * gq);
                bv0 = ld8f(w.vbar[l - 1] + off + 8 * gq);
                bv1 = ld8f(w.vbar[l - 1] + off + 32 + 8 * gq);
            }
            f32x4 ak[4] = {}, av[4] = {};
            for (int u = 0; u < 4; ++u) {
                const int i = 16 * a2 + 4 * wv + u;
                const long qb = ((long)gh * g.N + (long)i * BS) * D;
                stage_rows(lq, q, qb, true, lane);
                stage_rows(ld, dout, qb, true, lane);
                wave_lds_sync();
                const bf16x8 aq0 = *(const bf16x8*)(lq + nq * LDS_ROW + 8 * gq);
                const bf16x8 aq1 = *(const bf16x8*)(lq + nq * LDS_ROW + 32 + 8 * gq);
                const bf16x8 ad0 = *(const bf16x8*)(ld + nq * LDS_ROW + 8 * gq);
                const bf16x8 ad1 = *(const bf16x8*)(ld + nq * LDS_ROW + 32 + 8 * gq);
                f32x4 s = mfma32(aq1, bk1, mfma32(aq0, bk0, zero));  // S[query][entry]
                f32x4 dp = mfma32(ad1, bv1, mfma32(ad0, bv0, zero));
                const long tq = (long)gh * g.N + (long)i * BS + 4 * gq;
                const float4 l4 = *(const float4*)(lse + tq);
                const float4 d4 = *(const float4*)(w.delta + tq);
                const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
                bf16x4 pP, pS;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float P = ev ? fast_exp2(s[r] * c - lr[r] * LOG2E) : 0.f;
                    pP[r] = (bf16)P;
                    pS[r] = (bf16)(P * (dp[r] - dr[r]));
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
                    ak[d] = mfma16(lds_read_tr(lq + off), pS, ak[d]);
                    av[d] = mfma16(lds_read_tr(ld + off), pP, av[d]);
                }
                wave_lds_sync();
            }
            // reduce the four waves in a fixed order
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    red[wv][0][d][r][lane] = ak[d][r];
                    red[wv][1][d][r][lane] = av[d][r];
                }
            __syncthreads();
            for (int x = threadIdx.x; x < 2 * 4 * 4 * 64; x += blockDim.x) {
                const int kind = x >> 10, d = (x >> 8) & 3, r = (x >> 6) & 3, ln = x & 63;
                float s = red[0][kind][d][r][ln] + red[1][kind][d][r][ln] +
                          red[2][kind][d][r][ln] + red[3][kind][d][r][ln];
                const int ent = e0 + (ln & 15), dim = 16 * d + 4 * (ln >> 4) + r;
                if (ent < g.K) {
                    float* dst = w.part[l - 1] +
                                 ((((long)gh * g.n[2] + a2) * g.K + ent) * 2 + kind) * D;
                    dst[dim] = kind == 0 ? s * g.scale : s;
                }
            }
            __syncthreads();
        }
    }
}

// dbar_l[j] = sum over level-l query blocks a that chose j, and over the
// level-2 blocks under a, of the partial sums at j's slot in a's list.
__global__ __launch_bounds__(256) void enrich_sum(Geo g, Ws w, int l)
{
    const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (long)g.G * g.n[l] * D) return;
    const int dim = (int)(id % D);
    const long blk = id / D;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * g.K;
    const int span = 1 << (4 * (l - 2));  // level-2 blocks per level-l block
    float sk = 0.f, sv = 0.f;
    for (int e = rp[j]; e < rp[j + 1]; ++e) {
        const int a = cl[e];
        const int* sel = w.idx[l - 1] + ((long)gh * g.n[l] + a) * g.K;
        int lo = 0, hi = g.K - 1;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (sel[mid] < j) lo = mid + 1; else hi = mid;
        }
        for (int a2 = a * span; a2 < (a + 1) * span; ++a2) {
            const float* p = w.part[l - 1] + (((long)gh * g.n[2] + a2) * g.K + lo) * 2 * D;
            sk += p[dim];
            sv += p[D + dim];
        }
    }
    float* dst = w.dbar[l - 1] + ((long)gh * g.n[l] + j) * 2 * D;
    dst[dim] = sk;
    dst[D + dim] = sv;
}

__global__ __launch_bounds__(256) void dkdv_bf16(const unsigned short* __restrict__ q,
                                                 const unsigned short* __restrict__ k,
                                                 const unsigned short* __restrict__ v,
                                                 const float* __restrict__ lse,
                                                 const unsigned short* __restrict__ dout,
                                                 unsigned short* __restrict__ dk,
                                                 unsigned short* __restrict__ dv, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][4][TILE];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gq = lane >> 4, nq = lane & 15;
    const long kblk = (long)blockIdx.x * 4 + wv;
    if (kblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(kblk / g.n[1]), j = (int)(kblk % g.n[1]);
    const bool enrich = !(g.flags & LLSA_NO_ENRICH);
    const float c = g.scale * LOG2E;
    const long kbase = ((long)gh * g.N + (long)j * BS) * D;
    const bf16x8 bk0 = ld8(k + kbase + nq * D + 8 * gq), bk1 = ld8(k + kbase + nq * D + 32 + 8 * gq);
    const bf16x8 bv0 = ld8(v + kbase + nq * D + 8 * gq), bv1 = ld8(v + kbase + nq * D + 32 + 8 * gq);
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* list = w.col[0] + (long)gh * g.n[1] * g.K;
    const int beg = rp[j], end = rp[j + 1];
    unsigned short* lqa = smem[wv][0];
    unsigned short* lda = smem[wv][1];
    unsigned short* lqb = smem[wv][2];
    unsigned short* ldb = smem[wv][3];
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 zero = {};
    f32x4 accK[4] = {}, accV[4] = {};
    for (int e = beg; e < end; e += 2) {
        const bool hasb = e + 1 < end;
        const int ia = list[e], ib = hasb ? list[e + 1] : ia;
        const long qa = ((long)gh * g.N + (long)ia * BS) * D;
        const long qb = ((long)gh * g.N + (long)ib * BS) * D;
        stage_rows(lqa, q, qa, true, lane);
        stage_rows(lda, dout, qa, true, lane);
        stage_rows(lqb, q, qb, hasb, lane);
        stage_rows(ldb, dout, qb, hasb, lane);
        const long ta = (long)gh * g.N + (long)ia * BS + 4 * gq;
        const long tb = (long)gh * g.N + (long)ib * BS + 4 * gq;
        const float4 la4 = *(const float4*)(lse + ta), da4 = *(const float4*)(w.delta + ta);
        const float4 lb4 = *(const float4*)(lse + tb), db4 = *(const float4*)(w.delta + tb);
        wave_lds_sync();
        float P[2][4], S[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const unsigned short* lq = h ? lqb : lqa;
            const unsigned short* ld = h ? ldb : lda;
            const float4 l4 = h ? lb4 : la4, d4 = h ? db4 : da4;
            const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
            const bf16x8 aq0 = *(const bf16x8*)(lq + nq * LDS_ROW + 8 * gq);
            const bf16x8 aq1 = *(const bf16x8*)(lq + nq * LDS_ROW + 32 + 8 * gq);
            const bf16x8 ad0 = *(const bf16x8*)(ld + nq * LDS_ROW + 8 * gq);
            const bf16x8 ad1 = *(const bf16x8*)(ld + nq * LDS_ROW + 32 + 8 * gq);
            f32x4 s = mfma32(aq1, bk1, mfma32(aq0, bk0, zero));   // S[query 4gq+r][key nq]
            f32x4 dp = mfma32(ad1, bv1, mfma32(ad0, bv0, zero));  // dP[query][key]
            const bool live = h == 0 || hasb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float l2 = lr[r] * LOG2E;
                const float z = s[r] * c;
                float p = live ? fast_exp2(z - l2) : 0.f;
                float ds = p * (dp[r] - dr[r]);
                if (enrich) {  // level-1 pooled token of this key block
                    const float zm = row16_sum(z) * (1.0f / BS);
                    const float dpm = row16_sum(dp[r]) * (1.0f / BS);
                    const float pe = live ? fast_exp2(zm - l2) : 0.f;
                    p += pe * (1.0f / BS);
                    ds += pe * (dpm - dr[r]) * (1.0f / BS);
                }
                P[h][r] = p;
                S[h][r] = ds;
            }
        }
        bf16x8 bp, bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bp[r] = (bf16)P[0][r];
            bp[4 + r] = (bf16)P[1][r];
            bs[r] = (bf16)S[0][r];
            bs[4 + r] = (bf16)S[1][r];
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
            bf16x4 da = lds_read_tr(lda + off), db = lds_read_tr(ldb + off);
            bf16x4 qa4 = lds_read_tr(lqa + off), qb4 = lds_read_tr(lqb + off);
            bf16x8 adO = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3]};
            bf16x8 aQ = {qa4[0], qa4[1], qa4[2], qa4[3], qb4[0], qb4[1], qb4[2], qb4[3]};
            accV[d] = mfma32(adO, bp, accV[d]);
            accK[d] = mfma32(aQ, bs, accK[d]);
        }
        wave_lds_sync();
    }
    // epilogue: scale, add the pooled-level gradients (levels >= 2), store
    const long obase = kbase + nq * D + 4 * gq;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float xk[4], xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xk[r] = accK[d][r] * g.scale;
            xv[r] = accV[d][r];
        }
        if (enrich)
            for (int l = 2; l <= g.L; ++l) {
                const int a = j >> (4 * (l - 1));
                const float wgt = 1.0f / (float)(1 << (4 * l));
                const float* db = w.dbar[l - 1] + ((long)gh * g.n[l] + a) * 2 * D + 16 * d + 4 * gq;
                const float4 gk = *(const float4*)db, gv = *(const float4*)(db + D);
                xk[0] += gk.x * wgt; xk[1] += gk.y * wgt; xk[2] += gk.z * wgt; xk[3] += gk.w * wgt;
                xv[0] += gv.x * wgt; xv[1] += gv.y * wgt; xv[2] += gv.z * wgt; xv[3] += gv.w * wgt;
            }
        u16x4 ok, ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ok[r] = f2bf(xk[r]);
            ov[r] = f2bf(xv[r]);
        }
        *(u16x4*)(dk + obase + 16 * d) = ok;
        *(u16x4*)(dv + obase + 16 * d) = ov;
    }
}

// ------------------------------------------------------------ fp32 path

template <typename F>
__device__ __forceinline__ void for_each_entry(const Geo& g, const Ws& w, const float* k,
                                               const float* v, int gh, int t, F f)
{
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + t / BS) * g.K;
    for (int s = 0; s < g.K; ++s)
        for (int r = 0; r < BS; ++r) {
            long row = ((long)gh * g.N + (long)sel[s] * BS + r) * D;
            f(k + row, v + row);
        }
    if (!(g.flags & LLSA_NO_ENRICH))
        for (int lv = 1; lv <= g.L; ++lv) {
            const int a = t >> (4 * lv);
            const int* sl = w.idx[lv - 1] + ((long)gh * g.n[lv] + a) * g.K;
            for (int s = 0; s < g.K; ++s) {
                long row = ((long)gh * g.n[lv] + sl[s]) * D;
                f(w.kbar[lv - 1] + row, w.vbar[lv - 1] + row);
            }
        }
}

__global__ __launch_bounds__(256) void dq_f32(const float* __restrict__ q,
                                              const float* __restrict__ k,
                                              const float* __restrict__ v,
                                              const float* __restrict__ o,
                                              const float* __restrict__ lse,
                                              const float* __restrict__ dout,
                                              float* __restrict__ dq, Geo g, Ws w)
{
    const long tg = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (tg >= (long)g.G * g.N) return;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    const float* qr = q + tg * D;
    const float* dr = dout + tg * D;
    float Dt = 0.f;
    for (int c = 0; c < D; ++c) Dt = fmaf(dr[c], o[tg * D + c], Dt);
    w.delta[tg] = Dt;
    const float lt = lse[tg];
    float acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = 0.f;
    for_each_entry(g, w, k, v, gh, t, [&](const float* kr, const float* vr) {
        float z = 0.f, dp = 0.f;
        for (int c = 0; c < D; ++c) {
            z = fmaf(qr[c], kr[c], z);
            dp = fmaf(dr[c], vr[c], dp);
        }
        const float P = expf(z * g.scale - lt);
        const float ds = P * (dp - Dt) * g.scale;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, kr[c], acc[c]);
    });
#pragma unroll
    for (int c = 0; c < D; ++c) dq[tg * D + c] = acc[c];
}

// pooled-token gradients, every level: thread per (level block, channel)
__global__ __launch_bounds__(256) void enrich_f32(const float* __restrict__ q,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ dout, Geo g, Ws w,
                                                  int l)
{
    const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (long)g.G * g.n[l] * D) return;
    const int dim = (int)(id % D);
    const long blk = id / D;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    const float* kb = w.kbar[l - 1] + blk * D;
    const float* vb = w.vbar[l - 1] + blk * D;
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * g.K;
    const int span = 1 << (4 * l);
    float sk = 0.f, sv = 0.f;
    for (int e = rp[j]; e < rp[j + 1]; ++e) {
        const int a = cl[e];
        for (long t = (long)a * span; t < (long)(a + 1) * span; ++t) {
            const long tg = (long)gh * g.N + t;
            const float* qr = q + tg * D;
            const float* dr = dout + tg * D;
            float z = 0.f, dp = 0.f;
            for (int c = 0; c < D; ++c) {
                z = fmaf(qr[c], kb[c], z);
                dp = fmaf(dr[c], vb[c], dp);
            }
            const float P = expf(z * g.scale - lse[tg]);
            const float ds = P * (dp - w.delta[tg]);
            sk = fmaf(ds * g.scale, qr[dim], sk);
            sv = fmaf(P, dr[dim], sv);
        }
    }
    float* dst = w.dbar[l - 1] + blk * 2 * D;
    dst[dim] = sk;
    dst[D + dim] = sv;
}

__global__ __launch_bounds__(256) void dkdv_f32(const float* __restrict__ q,
                                                const float* __restrict__ k,
                                                const float* __restrict__ v,
                                                const float* __restrict__ lse,
                                                const float* __restrict__ dout,
                                                float* __restrict__ dk, float* __restrict__ dv,
                                                Geo g, Ws w)
{
    const long xg = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (xg >= (long)g.G * g.N) return;
    const int gh = (int)(xg / g.N), x = (int)(xg % g.N), j = x / BS;
    const float* kr = k + xg * D;
    const float* vr = v + xg * D;
    float ak[D], av[D];
#pragma unroll
    for (int c = 0; c < D; ++c) ak[c] = av[c] = 0.f;
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* cl = w.col[0] + (long)gh * g.n[1] * g.K;
    for (int e = rp[j]; e < rp[j + 1]; ++e)
        for (int r = 0; r < BS; ++r) {
            const long tg = (long)gh * g.N + (long)cl[e] * BS + r;
            const float* qr = q + tg * D;
            const float* dr = dout + tg * D;
            float z = 0.f, dp = 0.f;
            for (int c = 0; c < D; ++c) {
                z = fmaf(qr[c], kr[c], z);
                dp = fmaf(dr[c], vr[c], dp);
            }
            const float P = expf(z * g.scale - lse[tg]);
            const float ds = P * (dp - w.delta[tg]) * g.scale;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                ak[c] = fmaf(ds, qr[c], ak[c]);
                av[c] = fmaf(P, dr[c], av[c]);
            }
        }
    if (!(g.flags & LLSA_NO_ENRICH))
        for (int l = 1; l <= g.L; ++l) {
            const float wgt = 1.0f / (float)(1 << (4 * l));
            const float* db = w.dbar[l - 1] + ((long)gh * g.n[l] + (x >> (4 * l))) * 2 * D;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                ak[c] += db[c] * wgt;
                av[c] += db[D + c] * wgt;
            }
        }
#pragma unroll
    for (int c = 0; c < D; ++c) {
        dk[xg * D + c] = ak[c];
        dv[xg * D + c] = av[c];
    }
}

}  // namespace

hipError_t launch_attn_dq(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, int dtype, const Geo& g,
                          const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        hipLaunchKernelGGL(dq_bf16, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, (const unsigned short*)out, lse,
                           (const unsigned short*)dout, (unsigned short*)dq, g, w);
    } else {
        long ntok = (long)g.G * g.N;
        hipLaunchKernelGGL(dq_f32, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, (const float*)out,
                           lse, (const float*)dout, (float*)dq, g, w);
    }
    return hipGetLastError();
}

// Gradients of the pooled tokens (bf16: levels >= 2, level 1 being folded
// into the fine tiles; fp32: every level).  Needs delta from the dq pass.
hipError_t launch_attn_enrich(const void* q, const float* lse, const void* dout, int dtype,
                              const Geo& g, const Ws& w, hipStream_t st)
{
    if (g.flags & LLSA_NO_ENRICH) return hipSuccess;
    if (dtype == LLSA_BF16) {
        if (g.L < 2) return hipSuccess;
        hipLaunchKernelGGL(enrich_bwd_bf16, dim3(g.G * g.n[2]), dim3(256), 0, st,
                           (const unsigned short*)q, lse, (const unsigned short*)dout, g, w);
        hipError_t e = hipGetLastError();
        for (int l = 2; l <= g.L && e == hipSuccess; ++l) {
            long n = (long)g.G * g.n[l] * D;
            hipLaunchKernelGGL(enrich_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                               g, w, l);
            e = hipGetLastError();
        }
        return e;
    }
    hipError_t e = hipSuccess;
    for (int l = 1; l <= g.L && e == hipSuccess; ++l) {
        long n = (long)g.G * g.n[l] * D;
        hipLaunchKernelGGL(enrich_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           (const float*)q, lse, (const float*)dout, g, w, l);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_attn_dkdv(const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, void* dk, void* dv, int dtype, const Geo& g,
                            const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        hipLaunchKernelGGL(dkdv_bf16, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, lse, (const unsigned short*)dout,
                           (unsigned short*)dk, (unsigned short*)dv, g, w);
    } else {
        long ntok = (long)g.G * g.N;
        hipLaunchKernelGGL(dkdv_f32, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, lse,
                           (const float*)dout, (float*)dk, (float*)dv, g, w);
    }
    return hipGetLastError();
}

}  // namespace llsa
