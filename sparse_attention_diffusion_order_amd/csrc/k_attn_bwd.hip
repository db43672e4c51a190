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
//               pooled entries of every level as extra tiles (bf16-rounded
//               pyramid rows, as in the forward); also writes D.
//   enrich_bwd  one workgroup per level-2 block (256 query tokens): for each
//               level >= 2 entry list (shared by all 256 tokens) the partial
//               sums over the group, reduced across waves in fixed order.
//   enrich_sum  per pooled block: sum of the partials of the query groups
//               that chose it (found through that level's transpose).
//   dkdv_bf16   one wave per key block over its list T_1[j] (pairs of query
//               blocks form the 32-deep contraction); Q^T and dO^T read
//               transposed from LDS.  The level-1 pooled token of block j is
//               chosen by exactly the query blocks in T_1[j]: its logit and
//               dP come from an MFMA against the pooled row broadcast to all
//               16 columns, and since it averages the block's 16 keys its P/16
//               and dS/16 are added to every key column.  The epilogue adds
//               the pooled-level gradients of levels >= 2.
// fp32 path: plain VALU kernels with explicit pooled tokens at every level.
// No floating-point atomics anywhere: results are bit-identical run to run.
#include "common.h"

namespace llsa {
namespace {

// Staged 16-row tiles in LDS: 160-byte rows where a tile is read back
// transposed (ds_read_b64_tr_b16), 144-byte rows where it is only read as an
// MFMA operand (ds_read_b128); either way the accesses spread over all banks.
constexpr int LDS_ROW = 80;
constexpr int ROW_A = 72;
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

// Pooled entry e (0 .. L*K-1) of query block i: level 1 + e / K, slot e % K.
__device__ __forceinline__ long enrich_row(const Geo& g, const Ws& w, int gh, int i, int e,
                                           int* level)
{
    int l = 1 + e / g.K, s = e % g.K;
    int a = i >> (4 * (l - 1));
    int j = w.idx[l - 1][((long)gh * g.n[l] + a) * g.K + s];
    *level = l;
    return ((long)gh * g.n[l] + j) * D;
}

// Pooled-entry tile t for dq: pooled key rows staged row-major in LDS (for
// the transposed K^T read), A operands of S^T (pooled keys) and dP^T (pooled
// values) in registers; zeros for masked entries.
__device__ __forceinline__ int dq_tile(const Geo& g, const Ws& w, int gh, int i, int t,
                                       unsigned short* lds, bf16x8& k0, bf16x8& k1,
                                       bf16x8& v0, bf16x8& v1, int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    const int e0 = t * BS;
    const int nvalid = max(0, min(BS, g.L * g.K - e0));
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

// Registers of one prefetched pair of fine tiles for dq: rows vr and vr+8
// (columns vc .. vc+7) of the key and value tiles a and b -- 8 whole
// 128-byte rows per load instruction.
struct DqPair {
    bf16x8 kra0, kra1, krb0, krb1;
    bf16x8 vra0, vra1, vrb0, vrb1;
};

__device__ __forceinline__ void load_dq_fine(DqPair& f, const unsigned short* k,
                                             const unsigned short* v, long hbase, int ja, int jb,
                                             int lane)
{
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    const long a = hbase + (long)ja * BS * D + sr * D + sc;
    const long b = hbase + (long)max(jb, 0) * BS * D + sr * D + sc;
    f.kra0 = ld8(k + a);
    f.kra1 = ld8(k + a + 8 * D);
    f.vra0 = ld8(v + a);
    f.vra1 = ld8(v + a + 8 * D);
    f.krb0 = ld8(k + b);
    f.krb1 = ld8(k + b + 8 * D);
    f.vrb0 = ld8(v + b);
    f.vrb1 = ld8(v + b + 8 * D);
}

template <int ROW>
__device__ __forceinline__ void put_rows_s(unsigned short* lds, bf16x8 r0, bf16x8 r1, int lane)
{
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    *(bf16x8*)(lds + sr * ROW + sc) = r0;
    *(bf16x8*)(lds + (sr + 8) * ROW + sc) = r1;
}

__device__ __forceinline__ void put_rows(unsigned short* lds, bf16x8 r0, bf16x8 r1, int lane)
{
    put_rows_s<LDS_ROW>(lds, r0, r1, lane);
}

// dQ^T += K^T dS^T over two 16-entry tiles.  Key rows are in LDS (la, lb);
// ka*/kb* are the A operands of S^T (the same rows), va*/vb* those of dP^T.
// na / nb: valid entries (MASK == false: both tiles full).
template <bool MASK>
__device__ __forceinline__ void dq_pair(f32x4 (&acc)[4], bf16x8 bq0, bf16x8 bq1, bf16x8 bd0,
                                        bf16x8 bd1, float nl2, float Dq, bf16x8 ka0, bf16x8 ka1,
                                        bf16x8 kb0, bf16x8 kb1, bf16x8 va0, bf16x8 va1,
                                        bf16x8 vb0, bf16x8 vb1, const unsigned short* la,
                                        const unsigned short* lb, int na, int nb, float c,
                                        int lane)
{
    const int gq = lane >> 4;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 zero = {};
    const f32x4 sa = mfma32(ka1, bq1, mfma32(ka0, bq0, zero));
    const f32x4 sb = mfma32(kb1, bq1, mfma32(kb0, bq0, zero));
    const f32x4 pa = mfma32(va1, bd1, mfma32(va0, bd0, zero));  // dP^T
    const f32x4 pb = mfma32(vb1, bd1, mfma32(vb0, bd0, zero));
    bf16x8 bs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float Pa = fast_exp2(fmaf(sa[r], c, nl2));
        float Pb = fast_exp2(fmaf(sb[r], c, nl2));
        if (MASK) {
            Pa = (4 * gq + r < na) ? Pa : 0.f;
            Pb = (4 * gq + r < nb) ? Pb : 0.f;
        }
        bs[r] = (bf16)(Pa * (pa[r] - Dq));
        bs[4 + r] = (bf16)(Pb * (pb[r] - Dq));
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
        bf16x4 x0 = lds_read_tr(la + off), x1 = lds_read_tr(lb + off);
        bf16x8 ak = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        acc[d] = mfma32(ak, bs, acc[d]);
    }
}

__global__ __launch_bounds__(256) void dq_bf16(const unsigned short* __restrict__ q,
                                               const unsigned short* __restrict__ k,
                                               const unsigned short* __restrict__ v,
                                               const unsigned short* __restrict__ o,
                                               const float* __restrict__ lse,
                                               const unsigned short* __restrict__ dout,
                                               unsigned short* __restrict__ dq, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][4][TILE];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)xcd_block(blockIdx.x, gridDim.x) * 4 + wv;
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const bool enrich = !(g.flags & LLSA_NO_ENRICH);
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const long rowq = hbase + ((long)i * BS + nq) * D;
    const bf16x8 bq0 = ld8(q + rowq + 8 * gq), bq1 = ld8(q + rowq + 32 + 8 * gq);
    const bf16x8 bd0 = ld8(dout + rowq + 8 * gq), bd1 = ld8(dout + rowq + 32 + 8 * gq);
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i) * g.K;
    const int myj = lane < g.K ? sel[lane] : -1;
    float Dq;
    {
        const bf16x8 o0 = ld8(o + rowq + 8 * gq), o1 = ld8(o + rowq + 32 + 8 * gq);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += (float)bd0[e] * (float)o0[e] + (float)bd1[e] * (float)o1[e];
        Dq = sum_x4(s);
    }
    const long tok = (long)gh * g.N + (long)i * BS + nq;
    if (gq == 0) w.delta[tok] = Dq;
    const float nl2 = -lse[tok] * LOG2E;

    f32x4 acc[4] = {};
    unsigned short* la = smem[wv][0];
    unsigned short* lb = smem[wv][1];
    auto jsel = [&](int t) { return __builtin_amdgcn_readlane(myj, min(t, g.K - 1)); };
    unsigned short* lva = smem[wv][2];  // value tiles, read as operands only
    unsigned short* lvb = smem[wv][3];
    auto step = [&](const DqPair& f, bool full) {
        put_rows(la, f.kra0, f.kra1, lane);
        put_rows(lb, f.krb0, f.krb1, lane);
        put_rows_s<ROW_A>(lva, f.vra0, f.vra1, lane);
        put_rows_s<ROW_A>(lvb, f.vrb0, f.vrb1, lane);
        lds_fence();
        const bf16x8 ka0 = *(const bf16x8*)(la + nq * LDS_ROW + 8 * gq);
        const bf16x8 ka1 = *(const bf16x8*)(la + nq * LDS_ROW + 32 + 8 * gq);
        const bf16x8 kb0 = *(const bf16x8*)(lb + nq * LDS_ROW + 8 * gq);
        const bf16x8 kb1 = *(const bf16x8*)(lb + nq * LDS_ROW + 32 + 8 * gq);
        const bf16x8 va0 = *(const bf16x8*)(lva + nq * ROW_A + 8 * gq);
        const bf16x8 va1 = *(const bf16x8*)(lva + nq * ROW_A + 32 + 8 * gq);
        const bf16x8 vb0 = *(const bf16x8*)(lvb + nq * ROW_A + 8 * gq);
        const bf16x8 vb1 = *(const bf16x8*)(lvb + nq * ROW_A + 32 + 8 * gq);
        if (full)
            dq_pair<false>(acc, bq0, bq1, bd0, bd1, nl2, Dq, ka0, ka1, kb0, kb1, va0, va1, vb0,
                           vb1, la, lb, BS, BS, c, lane);
        else
            dq_pair<true>(acc, bq0, bq1, bd0, bd1, nl2, Dq, ka0, ka1, kb0, kb1, va0, va1, vb0,
                          vb1, la, lb, BS, 0, c, lane);
    };
    // fine tiles two per step, next pair prefetched; unconditional (clamped)
    // prefetches keep the compiler's wait counts exact
    if (g.K == 1) {
        DqPair A;
        load_dq_fine(A, k, v, hbase, jsel(0), jsel(0), lane);
        step(A, false);
    } else {
        const int npairs = g.K / 2;
        DqPair A, B;
        load_dq_fine(A, k, v, hbase, jsel(0), jsel(1), lane);
        for (int p = 0;; p += 2) {
            load_dq_fine(B, k, v, hbase, jsel(2 * p + 2), jsel(2 * p + 3), lane);
            step(A, true);
            if (p + 1 >= npairs) break;
            load_dq_fine(A, k, v, hbase, jsel(2 * p + 4), jsel(2 * p + 5), lane);
            step(B, true);
            if (p + 2 >= npairs) break;
        }
    }
    if (enrich) {  // pooled tokens of every level
        const int nt = (g.L * g.K + BS - 1) / BS;
        for (int t = 0; t < nt; t += 2) {
            bf16x8 ka0, ka1, va0, va1, kb0, kb1, vb0, vb1;
            int na = dq_tile(g, w, gh, i, t, la, ka0, ka1, va0, va1, lane);
            int nb = dq_tile(g, w, gh, i, t + 1, lb, kb0, kb1, vb0, vb1, lane);
            lds_fence();
            dq_pair<true>(acc, bq0, bq1, bd0, bd1, nl2, Dq, ka0, ka1, kb0, kb1, va0, va1, vb0,
                          vb1, la, lb, na, nb, c, lane);
        }
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
// level-2 blocks under a, of the partial sums at j's slot in a's list.  One
// wave per pooled block, lane = channel; list entries in ascending order.
__global__ __launch_bounds__(256) void enrich_sum(Geo g, Ws w, int l)
{
    const long blk = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (long)g.G * g.n[l]) return;
    const int dim = threadIdx.x & 63;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * g.K;
    const unsigned char* sl = w.slot[l - 1] + (long)gh * g.n[l] * g.K;
    const int span = 1 << (4 * (l - 2));  // level-2 blocks per level-l block
    const float* part = w.part[l - 1] + (long)gh * g.n[2] * g.K * 2 * D + dim;
    float sk = 0.f, sv = 0.f;
    const int beg = uniform(rp[j]), end = uniform(rp[j + 1]);
    // list entries in batches of 64: lane e holds entry beg + e (row offset
    // into the partials); then the batch's partial rows are summed in order
    for (int e0 = beg; e0 < end; e0 += 64) {
        const int ne = min(64, end - e0);
        const int lane = threadIdx.x & 63;
        int off = 0;  // in rows of 2*D floats
        if (lane < ne) off = cl[e0 + lane] * span * g.K + sl[e0 + lane];
        for (int e = 0; e < ne; ++e) {
            const long o = (long)__builtin_amdgcn_readlane(off, e) * 2 * D;
            for (int a2 = 0; a2 < span; ++a2) {
                const float* p = part + o + (long)a2 * g.K * 2 * D;
                sk += p[0];
                sv += p[D];
            }
        }
    }
    float* dst = w.dbar[l - 1] + blk * 2 * D;
    dst[dim] = sk;
    dst[D + dim] = sv;
}

// Registers of one prefetched pair of query blocks for dk/dv: the q and dout
// rows this lane stages into LDS, and the per-row lse / delta of the rows
// 4(lane/16) .. +3 it needs for P and dS.
struct QPair {
    bf16x8 qa0, qa1, da0, da1, qb0, qb1, db0, db1;
    float4 la4, lb4, ea4, eb4;
};

__device__ __forceinline__ void load_qpair(QPair& f, const unsigned short* q,
                                           const unsigned short* dout, const float* lse,
                                           const float* delta, long hbase, long tbase, int ia,
                                           int ib, int lane)
{
    const int gq = lane >> 4;
    const int sr = lane >> 3, sc = (lane & 7) * 8;
    const long a = hbase + (long)ia * BS * D;
    const long b = hbase + (long)ib * BS * D;
    f.qa0 = ld8(q + a + sr * D + sc);
    f.qa1 = ld8(q + a + (sr + 8) * D + sc);
    f.da0 = ld8(dout + a + sr * D + sc);
    f.da1 = ld8(dout + a + (sr + 8) * D + sc);
    f.qb0 = ld8(q + b + sr * D + sc);
    f.qb1 = ld8(q + b + (sr + 8) * D + sc);
    f.db0 = ld8(dout + b + sr * D + sc);
    f.db1 = ld8(dout + b + (sr + 8) * D + sc);
    f.la4 = *(const float4*)(lse + tbase + (long)ia * BS + 4 * gq);
    f.ea4 = *(const float4*)(delta + tbase + (long)ia * BS + 4 * gq);
    f.lb4 = *(const float4*)(lse + tbase + (long)ib * BS + 4 * gq);
    f.eb4 = *(const float4*)(delta + tbase + (long)ib * BS + 4 * gq);
}

// P and dS of one query block (rows in LDS at lq / ld) against this wave's
// key block; lane holds rows 4(lane/16)+r, key lane%16.  With enrichment the
// block's level-1 pooled token (kp*, vp*: its row in every column) adds P/16
// and dS/16 to each key.
__device__ __forceinline__ void kv_block(const unsigned short* lq, const unsigned short* ld,
                                         float4 l4, float4 d4, bool live, bf16x8 bk0,
                                         bf16x8 bk1, bf16x8 bv0, bf16x8 bv1, bool enrich,
                                         bf16x8 kp0, bf16x8 kp1, bf16x8 vp0, bf16x8 vp1,
                                         float c, int lane, float (&P)[4], float (&S)[4])
{
    const int gq = lane >> 4, nq = lane & 15;
    const f32x4 zero = {};
    const bf16x8 aq0 = *(const bf16x8*)(lq + nq * LDS_ROW + 8 * gq);
    const bf16x8 aq1 = *(const bf16x8*)(lq + nq * LDS_ROW + 32 + 8 * gq);
    const bf16x8 ad0 = *(const bf16x8*)(ld + nq * LDS_ROW + 8 * gq);
    const bf16x8 ad1 = *(const bf16x8*)(ld + nq * LDS_ROW + 32 + 8 * gq);
    const f32x4 s = mfma32(aq1, bk1, mfma32(aq0, bk0, zero));   // S[query 4gq+r][key nq]
    const f32x4 dp = mfma32(ad1, bv1, mfma32(ad0, bv0, zero));  // dP[query][key]
    f32x4 se = zero, dpe = zero;
    if (enrich) {
        se = mfma32(aq1, kp1, mfma32(aq0, kp0, zero));   // pooled logit, every column
        dpe = mfma32(ad1, vp1, mfma32(ad0, vp0, zero));
    }
    const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float nl2 = -lr[r] * LOG2E;
        float p = live ? fast_exp2(fmaf(s[r], c, nl2)) : 0.f;
        float ds = p * (dp[r] - dr[r]);
        if (enrich) {
            const float pe = live ? fast_exp2(fmaf(se[r], c, nl2)) : 0.f;
            p += pe * (1.0f / BS);
            ds += pe * (dpe[r] - dr[r]) * (1.0f / BS);
        }
        P[r] = p;
        S[r] = ds;
    }
}

__global__ __launch_bounds__(256, 2) void dkdv_bf16(const unsigned short* __restrict__ q,
                                                 const unsigned short* __restrict__ k,
                                                 const unsigned short* __restrict__ v,
                                                 const float* __restrict__ lse,
                                                 const unsigned short* __restrict__ dout,
                                                 unsigned short* __restrict__ dk,
                                                 unsigned short* __restrict__ dv, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][4][TILE];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const long kblk = (long)xcd_block(blockIdx.x, gridDim.x) * 4 + wv;
    if (kblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(kblk / g.n[1]), j = (int)(kblk % g.n[1]);
    const bool enrich = !(g.flags & LLSA_NO_ENRICH);
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const long tbase = (long)gh * g.N;
    const long kbase = hbase + (long)j * BS * D;
    const bf16x8 bk0 = ld8(k + kbase + nq * D + 8 * gq), bk1 = ld8(k + kbase + nq * D + 32 + 8 * gq);
    const bf16x8 bv0 = ld8(v + kbase + nq * D + 8 * gq), bv1 = ld8(v + kbase + nq * D + 32 + 8 * gq);
    bf16x8 kp0 = {}, kp1 = {}, vp0 = {}, vp1 = {};  // level-1 pooled row, in every column
    if (enrich) {
        const long prow = ((long)gh * g.n[1] + j) * D;
        kp0 = ld8f(w.kbar[0] + prow + 8 * gq);
        kp1 = ld8f(w.kbar[0] + prow + 32 + 8 * gq);
        vp0 = ld8f(w.vbar[0] + prow + 8 * gq);
        vp1 = ld8f(w.vbar[0] + prow + 32 + 8 * gq);
    }
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* list = w.col[0] + (long)gh * g.n[1] * g.K;
    const int beg = uniform(rp[j]), end = uniform(rp[j + 1]);
    unsigned short* lqa = smem[wv][0];
    unsigned short* lda = smem[wv][1];
    unsigned short* lqb = smem[wv][2];
    unsigned short* ldb = smem[wv][3];
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 zero = {};
    f32x4 accK[4] = {}, accV[4] = {};
    // A missing second block of the last pair re-reads the first one (valid
    // memory); its P and dS are zeroed, so it contributes nothing.  Two
    // register sets alternate so the next pair's loads fly during this one.
    auto step = [&](const QPair& f, bool hasb) {
        put_rows(lqa, f.qa0, f.qa1, lane);
        put_rows(lda, f.da0, f.da1, lane);
        put_rows(lqb, f.qb0, f.qb1, lane);
        put_rows(ldb, f.db0, f.db1, lane);
        lds_fence();
        float Pa[4], Sa[4], Pb[4], Sb[4];
        kv_block(lqa, lda, f.la4, f.ea4, true, bk0, bk1, bv0, bv1, enrich, kp0, kp1, vp0, vp1,
                 c, lane, Pa, Sa);
        kv_block(lqb, ldb, f.lb4, f.eb4, hasb, bk0, bk1, bv0, bv1, enrich, kp0, kp1, vp0, vp1,
                 c, lane, Pb, Sb);
        bf16x8 bp, bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bp[r] = (bf16)Pa[r];
            bp[4 + r] = (bf16)Pb[r];
            bs[r] = (bf16)Sa[r];
            bs[4 + r] = (bf16)Sb[r];
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
    };
    auto fetch = [&](QPair& f, int e) {
        load_qpair(f, q, dout, lse, w.delta, hbase, tbase, list[min(e, end - 1)],
                   list[min(e + 1, end - 1)], lane);
    };
    QPair A, B;
    if (beg < end) {
        fetch(A, beg);
        for (int e = beg;; e += 4) {
            fetch(B, e + 2);  // unconditional (clamped): exact wait counts
            step(A, e + 1 < end);
            if (e + 2 >= end) break;
            fetch(A, e + 4);
            step(B, e + 3 < end);
            if (e + 4 >= end) break;
        }
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

// Gradients of the pooled tokens (bf16: levels >= 2, level 1 being handled in
// the dk/dv pass; fp32: every level).  Needs delta from the dq pass.
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
            long n = (long)g.G * g.n[l];
            hipLaunchKernelGGL(enrich_sum, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, g, w,
                               l);
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
