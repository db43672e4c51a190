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
//               pooled entries of every level as extra tiles (the bf16
//               pyramid copy, as in the forward); also writes D.
//   enrich_bwd  one workgroup per level-2 block (256 query tokens): for each
//               level >= 2 entry list (shared by all 256 tokens) the partial
//               sums over the group, reduced across waves in fixed order.
//   enrich_sum  per pooled block: sum of the partials of the query groups
//               that chose it (found through that level's transpose).
//   dkdv_bf16   one wave per key block over its list T_1[j], one query block
//               per step; Q^T and dO^T read transposed from LDS.  The level-1
//               pooled token of block j is chosen by exactly the query blocks
//               in T_1[j]; it averages the block's 16 keys, so its P/16 and
//               dS/16 (stored by the dq pass) are added to every key column.
//               The epilogue adds the pooled-level gradients of levels >= 2.
// fp32 path: plain VALU kernels, one wave per row (lane = channel), with
// explicit pooled tokens at every level.
// No floating-point atomics anywhere: results are bit-identical run to run.
#include "common.h"
#include "transpose.h"

namespace llsa {
namespace {

// Staged 16-row tiles in LDS (TileShape<D>): rows of D + 16 elements where a
// tile is read back transposed (ds_read_b64_tr_b16), D + 8 where it is only
// read as an MFMA operand (ds_read_b128); either way the accesses spread over
// all banks.
template <int D>
constexpr int TILE = BS * TileShape<D>::ROW_T;

__device__ __forceinline__ bf16x8 ld8(const unsigned short* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ bf16x8 ld8f(const float* p)
{
    float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    bf16x8 r;
    r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
    r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
    return r;
}


// Registers of one prefetched pair of fine tiles for dq: load u holds row
// sr + RPI u (columns sc .. sc+7) of the key and value tiles a and b -- whole
// rows, 1024 bytes per load instruction.
template <int D>
struct DqPair {
    static constexpr int NI = TileShape<D>::NI;
    bf16x8 kra[NI], krb[NI], vra[NI], vrb[NI];
};

// a tile (TileShape<D> chunks) into LDS rows read back transposed
template <int D>
__device__ __forceinline__ void put_rows(unsigned short* lds, const bf16x8 (&r)[TileShape<D>::NI],
                                         int lane)
{
    stage_rows<D, TileShape<D>::ROW_T>(lds, r, lane);
}

// dQ^T += K^T dS^T over two 16-entry tiles.  Key rows are in LDS (la, lb);
// ka*/kb* are the A operands of S^T (the same rows), va*/vb* those of dP^T.
// na / nb: valid entries (MASK == false: both tiles full).
// ba / bb (MASK only, may be null): logit bias of rows 4(lane/16) + r of
// tiles a and b (log2 units; pooled entries under the size-weighted variant).
// pe != nullptr: entries ea + 4(lane/16) + r (tile a) and ea + 16 + ... (tile
// b) below K1 are level-1 pooled tokens; their P and dS are stored at
// pe[entry][0 | 1][query] for the key-major dk/dv pass.
template <bool MASK, int D>
__device__ __forceinline__ void dq_pair(f32x4 (&acc)[D / 16], const bf16x8 (&bq)[D / 32],
                                        const bf16x8 (&bd)[D / 32], float nl2, float Dq,
                                        const bf16x8 (&ka)[D / 32], const bf16x8 (&kb)[D / 32],
                                        const bf16x8 (&va)[D / 32], const bf16x8 (&vb)[D / 32],
                                        const unsigned short* la, const unsigned short* lb,
                                        int na, int nb, float c, int lane, float* pe = nullptr,
                                        int ea = 0, int K1 = 0, const float* ba = nullptr,
                                        const float* bb = nullptr)
{
    const int gq = lane >> 4;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 sa = scores<D>(ka, bq);
    const f32x4 sb = scores<D>(kb, bq);
    const f32x4 pa = scores<D>(va, bd);  // dP^T
    const f32x4 pb = scores<D>(vb, bd);
    bf16x8 bs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float xa = (MASK && ba) ? ba[r] : 0.f, xb = (MASK && bb) ? bb[r] : 0.f;
        float Pa = fast_exp2(fmaf(sa[r], c, nl2 + xa));
        float Pb = fast_exp2(fmaf(sb[r], c, nl2 + xb));
        if (MASK) {
            Pa = (4 * gq + r < na) ? Pa : 0.f;
            Pb = (4 * gq + r < nb) ? Pb : 0.f;
        }
        const float dSa = Pa * (pa[r] - Dq), dSb = Pb * (pb[r] - Dq);
        if (pe) {
            const int nq = lane & 15;
            const int e_a = ea + 4 * gq + r, e_b = e_a + BS;
            if (e_a < K1) {
                pe[e_a * 2 * BS + nq] = Pa;
                pe[e_a * 2 * BS + BS + nq] = dSa;
            }
            if (e_b < K1) {
                pe[e_b * 2 * BS + nq] = Pb;
                pe[e_b * 2 * BS + BS + nq] = dSb;
            }
        }
        bs[r] = (bf16)dSa;
        bs[4 + r] = (bf16)dSb;
    }
#pragma unroll
    for (int d = 0; d < D / 16; ++d) {
        const int off = (4 * gq + rr) * TileShape<D>::ROW_T + 16 * d + 4 * xx;
        bf16x4 x0 = lds_read_tr(la + off), x1 = lds_read_tr(lb + off);
        bf16x8 ak = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        acc[d] = mfma32(ak, bs, acc[d]);
    }
}

constexpr int MAX_E = MAX_L * 64;  // pooled entries per query block (sum of the levels' K)

// Per-wave LDS of dq: two key tiles (160-byte rows, read as operands and
// transposed), two value tiles (144-byte rows) and the pooled-entry table.
template <int ECAP, int D>
struct DqLds {
    static constexpr int K_TILE = BS * TileShape<D>::ROW_T;
    static constexpr int V_TILE = BS * TileShape<D>::ROW_A;
    static constexpr int PER_WAVE = 2 * K_TILE + 2 * V_TILE + 2 * ECAP;
};

// at least two waves per SIMD at d = 128 (d = 64 has three without a bound)
// One workgroup of the dQ pass: workgroup bid of nb (XCD-aware order).
template <int ECAP, int D>
__device__ __forceinline__ void dq_block(const unsigned short* __restrict__ q,
                                         const unsigned short* __restrict__ k,
                                         const unsigned short* __restrict__ v,
                                         const unsigned short* __restrict__ o,
                                         const float* __restrict__ lse,
                                         const unsigned short* __restrict__ dout,
                                         unsigned short* __restrict__ dq, const Geo& g,
                                         const Ws& w, int bid, int nb)
{
    using Lay = DqLds<ECAP, D>;
    using TS = TileShape<D>;
    constexpr int NI = TS::NI;
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][Lay::PER_WAVE];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)xcd_block(bid, nb) * 4 + wv;
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const long rowq = hbase + ((long)i * BS + nq) * D;
    bf16x8 bq[NI], bd[NI];  // query and dO rows lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        bq[u] = ld8(q + rowq + 32 * u + 8 * gq);
        bd[u] = ld8(dout + rowq + 32 * u + 8 * gq);
    }
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i) * g.K;
    const int myj = lane < g.K ? sel[lane] : 0;
    float Dq;
    {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const bf16x8 ou = ld8(o + rowq + 32 * u + 8 * gq);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += (float)bd[u][e] * (float)ou[e];
        }
        Dq = sum_x4(s);
    }
    const long tok = (long)gh * g.N + (long)i * BS + nq;
    if (gq == 0) w.delta[tok] = Dq;
    const float nl2 = -lse[tok] * LOG2E;
    // pooled entries e = (l - l0) * K + slot of the enriching levels l0..L:
    // their rows in the bf16 pooled arrays
    const int E = g.n_pooled();
    int* ent = (int*)(smem[wv] + 2 * Lay::K_TILE + 2 * Lay::V_TILE);
    for (int l = g.l0; l <= g.L; ++l) {
        const int Kl = g.Kl[l];
        const long a = (long)gh * g.n[l] + (i >> (4 * (l - 1)));
        for (int s0 = 0; s0 < Kl; s0 += 64)
            if (s0 + lane < Kl)
                ent[g.eoff[l] + s0 + lane] =
                    (int)(w.prow[l - 1] + (long)gh * g.n[l] + w.idx[l - 1][a * Kl + s0 + lane]);
    }
    lds_fence();

    f32x4 acc[D / 16] = {};
    unsigned short* la = smem[wv];  // key tiles
    unsigned short* lb = la + Lay::K_TILE;
    unsigned short* lva = lb + Lay::K_TILE;  // value tiles, read as operands only
    unsigned short* lvb = lva + Lay::V_TILE;
    // one pipeline over NF fine pairs then the pooled pairs, next pair in
    // flight; unconditional (clamped) loads keep the wait counts exact
    const int NF = (g.K + 1) / 2;
    const int NT = (E + BS - 1) / BS;
    const int NP = NF + (NT + 1) / 2;
    const int sr = lane / TS::LPR, sc = (lane % TS::LPR) * 8;
    auto load_pair = [&](DqPair<D>& f, int p) {
        long ka[NI], kb[NI];  // element offsets of row sr + RPI u of tiles a and b
        const unsigned short *kp, *vp;
        if (p < NF) {
            const int ja = __builtin_amdgcn_readlane(myj, min(2 * p, g.K - 1));
            const int jb = __builtin_amdgcn_readlane(myj, min(2 * p + 1, g.K - 1));
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                ka[u] = hbase + ((long)ja * BS + sr + TS::RPI * u) * D + sc;
                kb[u] = hbase + ((long)jb * BS + sr + TS::RPI * u) * D + sc;
            }
            kp = k;
            vp = v;
        } else {  // pooled pairs exist only when E > 0
            const int t = 2 * (p - NF);
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                ka[u] = (long)ent[min(BS * t + sr + TS::RPI * u, E - 1)] * D + sc;
                kb[u] = (long)ent[min(BS * t + BS + sr + TS::RPI * u, E - 1)] * D + sc;
            }
            kp = w.kb16;
            vp = w.vb16;
        }
        // issue order: key rows, then value rows, of tile a, then of tile b
#pragma unroll
        for (int u = 0; u < NI; ++u) f.kra[u] = ld8(kp + ka[u]);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.vra[u] = ld8(vp + ka[u]);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.krb[u] = ld8(kp + kb[u]);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.vrb[u] = ld8(vp + kb[u]);
    };
    auto step = [&](const DqPair<D>& f, int p) {
        put_rows<D>(la, f.kra, lane);
        put_rows<D>(lb, f.krb, lane);
        stage_rows<D, TS::ROW_A>(lva, f.vra, lane);
        stage_rows<D, TS::ROW_A>(lvb, f.vrb, lane);
        lds_fence();
        bf16x8 ka[NI], kb[NI], va[NI], vb[NI];
        operand_rows<D, TS::ROW_T>(la, ka, lane);
        operand_rows<D, TS::ROW_T>(lb, kb, lane);
        operand_rows<D, TS::ROW_A>(lva, va, lane);
        operand_rows<D, TS::ROW_A>(lvb, vb, lane);
        if (p < NF && g.K > 1) {
            dq_pair<false, D>(acc, bq, bd, nl2, Dq, ka, kb, va, vb, la, lb, BS, BS, c, lane);
        } else {
            const int e0 = p < NF ? 0 : BS * 2 * (p - NF);
            const int na = p < NF ? BS : max(0, min(BS, E - e0));
            const int nb = p < NF ? 0 : max(0, min(BS, E - e0 - BS));
            const bool pooled = p >= NF;
            float* pe = (pooled && g.l0 == 1 && e0 < g.K)
                            ? w.pe1 + ((long)gh * g.n[1] + i) * g.K * 2 * BS : nullptr;
            float ba[4], bb[4];  // pooled rows: the logit bias of the entry's level
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ea = e0 + 4 * gq + r;
                ba[r] = pooled ? g.lb2 * (float)g.entry_level(ea) : 0.f;
                bb[r] = pooled ? g.lb2 * (float)g.entry_level(ea + BS) : 0.f;
            }
            dq_pair<true, D>(acc, bq, bd, nl2, Dq, ka, kb, va, vb, la, lb, na, nb, c, lane, pe,
                             e0, g.K, ba, bb);
        }
    };
    DqPair<D> A, B;
    load_pair(A, 0);
    for (int p = 0;; p += 2) {
        load_pair(B, min(p + 1, NP - 1));
        step(A, p);
        if (p + 1 >= NP) break;
        load_pair(A, min(p + 2, NP - 1));
        step(B, p + 1);
        if (p + 2 >= NP) break;
    }
    const long obase = rowq + 4 * gq;
#pragma unroll
    for (int d = 0; d < D / 16; ++d) {
        u16x4 r4;
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[r] = f2bf(acc[d][r] * g.scale);
        *(u16x4*)(dq + obase + 16 * d) = r4;
    }
}

template <int ECAP, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == D128 ? 2 : 1))) void dq_bf16(const unsigned short* __restrict__ q,
                                               const unsigned short* __restrict__ k,
                                               const unsigned short* __restrict__ v,
                                               const unsigned short* __restrict__ o,
                                               const float* __restrict__ lse,
                                               const unsigned short* __restrict__ dout,
                                               unsigned short* __restrict__ dq, Geo g, Ws w)
{
    dq_block<ECAP, D>(q, k, v, o, lse, dout, dq, g, w, blockIdx.x, gridDim.x);
}

// The dQ pass with the first transpose launch in front: workgroups below
// tr_pad (tr_wgs rounded up to a multiple of 8, so that the dQ workgroups keep
// their XCD placement) build the transpose's first levels, the rest run dQ.
// The two parts read only the forward's results and write disjoint workspace
// regions, so the latency-bound transpose overlaps dQ.
template <int ECAP, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == D128 ? 2 : 1))) void dq_tr_bf16(const unsigned short* __restrict__ q,
                                               const unsigned short* __restrict__ k,
                                               const unsigned short* __restrict__ v,
                                               const unsigned short* __restrict__ o,
                                               const float* __restrict__ lse,
                                               const unsigned short* __restrict__ dout,
                                               unsigned short* __restrict__ dq, Geo g, Ws w,
                                               TrFirst tr, int tr_pad)
{
    const int b = blockIdx.x;
    if (b < tr_pad) {
        if (b < tr.wgs) transpose_block(g, w, tr.l, tr.pair, b);
        return;
    }
    dq_block<ECAP, D>(q, k, v, o, lse, dout, dq, g, w, b - tr_pad, (int)gridDim.x - tr_pad);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == D128 ? 2 : 1))) void enrich_bwd_bf16(const unsigned short* __restrict__ q,
                                                       const float* __restrict__ lse,
                                                       const unsigned short* __restrict__ dout,
                                                       Geo g, Ws w)
{
    using TS = TileShape<D>;
    constexpr int NI = TS::NI, ND = D / 16;
    // per-wave Q and dO tiles; after the last tile the same memory holds the
    // four waves' partial sums for the cross-wave reduction
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][2][TILE<D>];
    // lse and delta of each wave's 64 queries (its four blocks are consecutive),
    // loaded once, so no step waits on a global load for them
    __shared__ __attribute__((aligned(16))) float rowst[4][2][4 * BS];
    float* red = (float*)&smem[0][0][0];  // [wave][dtile][r][lane], one kind at a time
    static_assert(sizeof(smem) >= 4 * ND * 4 * 64 * sizeof(float), "reduction buffer");
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gq = lane >> 4, nq = lane & 15;
    const int gh = blockIdx.x / g.n[2], a2 = blockIdx.x % g.n[2];
    const float c = g.scale * LOG2E;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const int sr = lane / TS::LPR, sc = (lane % TS::LPR) * 8;
    unsigned short* lq = smem[wv][0];
    unsigned short* ld = smem[wv][1];
    // this wave's four query blocks i = 16 a2 + 4 wv + u (u < 4); load v of
    // a block covers its row sr + RPI v
    auto row_addr = [&](int u) {
        const int i = 16 * a2 + 4 * wv + u;
        return ((long)gh * g.N + (long)i * BS + sr) * D + sc;
    };
    auto load_rows = [&](bf16x8 (&xq)[NI], bf16x8 (&xd)[NI], long a) {
#pragma unroll
        for (int v = 0; v < NI; ++v) xq[v] = ld8(q + a + (long)TS::RPI * v * D);
#pragma unroll
        for (int v = 0; v < NI; ++v) xd[v] = ld8(dout + a + (long)TS::RPI * v * D);
    };
    {
        const long t0 = (long)gh * g.N + (long)(16 * a2 + 4 * wv) * BS + lane;
        rowst[wv][0][lane] = lse[t0];
        rowst[wv][1][lane] = w.delta[t0];
    }
    for (int l = 2; l <= g.L; ++l) {
        const int al = a2 >> (4 * (l - 2));
        const int Kl = g.Kl[l];
        const int* sel = w.idx[l - 1] + ((long)gh * g.n[l] + al) * Kl;
        const float lb = g.lb2 * (float)l;  // size bias of a level-l token (log2)
        for (int e0 = 0; e0 < Kl; e0 += BS) {
            const bool ev = e0 + nq < Kl;
            bf16x8 bk[NI], bv[NI];  // entry rows lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
            for (int u = 0; u < NI; ++u) bk[u] = bv[u] = bf16x8{};
            if (ev) {
                long off = ((long)gh * g.n[l] + sel[e0 + nq]) * D;
#pragma unroll
                for (int u = 0; u < NI; ++u) {
                    bk[u] = ld8f(w.kbar[l - 1] + off + 32 * u + 8 * gq);
                    bv[u] = ld8f(w.vbar[l - 1] + off + 32 * u + 8 * gq);
                }
            }
            f32x4 ak[ND] = {}, av[ND] = {};
            // rows of block u + 1 are loaded while block u is computed
            bf16x8 xq[NI], xd[NI];
            load_rows(xq, xd, row_addr(0));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                put_rows<D>(lq, xq, lane);
                put_rows<D>(ld, xd, lane);
                load_rows(xq, xd, row_addr(min(u + 1, 3)));
                lds_fence();
                bf16x8 aq[NI], ad[NI];
                operand_rows<D, TS::ROW_T>(lq, aq, lane);
                operand_rows<D, TS::ROW_T>(ld, ad, lane);
                f32x4 s = scores<D>(aq, bk);  // S[query][entry]
                f32x4 dp = scores<D>(ad, bv);
                const float4 l4 = *(const float4*)&rowst[wv][0][u * BS + 4 * gq];
                const float4 d4 = *(const float4*)&rowst[wv][1][u * BS + 4 * gq];
                const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
                bf16x4 pP, pS;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float P = ev ? fast_exp2(s[r] * c - lr[r] * LOG2E + lb) : 0.f;
                    pP[r] = (bf16)P;
                    pS[r] = (bf16)(P * (dp[r] - dr[r]));
                }
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const int off = (4 * gq + rr) * TS::ROW_T + 16 * d + 4 * xx;
                    ak[d] = mfma16(lds_read_tr(lq + off), pS, ak[d]);
                    av[d] = mfma16(lds_read_tr(ld + off), pP, av[d]);
                }
            }
            // reduce the four waves in a fixed order, dk then dv
            for (int kind = 0; kind < 2; ++kind) {
                __syncthreads();  // tiles (or the previous kind) no longer read
#pragma unroll
                for (int d = 0; d < ND; ++d)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[((wv * ND + d) * 4 + r) * 64 + lane] = kind == 0 ? ak[d][r] : av[d][r];
                __syncthreads();
                for (int x = threadIdx.x; x < ND * 4 * 64; x += blockDim.x) {
                    const float s = red[x] + red[ND * 256 + x] + red[2 * ND * 256 + x] +
                                    red[3 * ND * 256 + x];
                    const int d = x >> 8, r = (x >> 6) & 3, ln = x & 63;
                    const int ent = e0 + (ln & 15), dim = 16 * d + 4 * (ln >> 4) + r;
                    if (ent < Kl) {
                        float* dst = w.part[l - 1] +
                                     ((((long)gh * g.n[2] + a2) * Kl + ent) * 2 + kind) * D;
                        dst[dim] = kind == 0 ? s * g.scale : s;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// dbar_l[j] = sum over level-l query blocks a that chose j, and over the
// level-2 blocks under a, of the partial sums at j's slot in a's list.  One
// wave per pooled block, lane = channels lane + 64 c; list entries in
// ascending order.
template <int D>
__global__ __launch_bounds__(256) void enrich_sum(Geo g, Ws w, int l)
{
    constexpr int NC = D / 64;  // channels dim + 64 c per lane
    const long blk = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (long)g.G * g.n[l]) return;
    const int dim = threadIdx.x & 63;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int Kl = g.Kl[l];
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * Kl;
    const unsigned char* sl = w.slot[l - 1] + (long)gh * g.n[l] * Kl;
    const int span = 1 << (4 * (l - 2));  // level-2 blocks per level-l block
    const float* part = w.part[l - 1] + (long)gh * g.n[2] * Kl * 2 * D + dim;
    float sk[NC] = {}, sv[NC] = {};
    const int beg = uniform(rp[j]), end = uniform(rp[j + 1]);
    // list entries in batches of 64: lane e holds entry beg + e (row offset
    // into the partials).  The batch's (entry, level-2 block) rows are summed
    // in order, eight loads in flight at a time.
    const int lane = threadIdx.x & 63;
    for (int e0 = beg; e0 < end; e0 += 64) {
        const int ne = min(64, end - e0);
        int off = 0;  // in rows of 2*D floats
        if (lane < ne) off = cl[e0 + lane] * span * Kl + sl[e0 + lane];
        const int nrow = ne * span;
        for (int q0 = 0; q0 < nrow; q0 += 8) {
            float vk[8][NC], vv[8][NC];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int qq = min(q0 + u, nrow - 1);
                const int e = qq / span, a2 = qq % span;
                const long o = ((long)__builtin_amdgcn_readlane(off, e) + (long)a2 * Kl) * 2 * D;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    vk[u][c] = part[o + 64 * c];
                    vv[u][c] = part[o + D + 64 * c];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < nrow)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        sk[c] += vk[u][c];
                        sv[c] += vv[u][c];
                    }
        }
    }
    float* dst = w.dbar[l - 1] + blk * 2 * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        dst[dim + 64 * c] = sk[c];
        dst[D + dim + 64 * c] = sv[c];
    }
}

// dk/dv: one wave (and workgroup) per key block j, over the query blocks of
// its list T_1[j], one block per step with the next one in flight.
//   S  = Q K^T, dP = dO V^T   (16x16x32 MFMA; lane holds query 4(lane/16)+r,
//                              key lane%16)
//   P = exp(s S - lse), dS = P (dP - D); when level 1 enriches, the level-1 pooled
//   token of block j (chosen by exactly the blocks of T_1[j]) adds P_e/16 and
//   dS_e/16 to every key column -- P_e and dS_e come from the dq pass
//   dV^T += dO^T P, dK^T += Q^T dS   (16x16x16 MFMA over the 16 queries;
//                                     Q^T, dO^T read transposed from LDS)
template <int D>
struct QBlock {
    bf16x8 q[D / 32], d[D / 32];  // load u: row sr + RPI u, channels sc .. sc+7
    float x;  // lane < 16: lse of row lane; < 32: delta of row lane - 16; else the
              // level-1 pooled P (lanes 32..47) and dS (48..63) of row lane % 16
};

template <int D>
__global__ __launch_bounds__(64) void dkdv_bf16(const unsigned short* __restrict__ q,
                                                const unsigned short* __restrict__ k,
                                                const unsigned short* __restrict__ v,
                                                const float* __restrict__ lse,
                                                const unsigned short* __restrict__ dout,
                                                unsigned short* __restrict__ dk,
                                                unsigned short* __restrict__ dv, Geo g, Ws w)
{
    using TS = TileShape<D>;
    constexpr int NI = TS::NI, ND = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned short lq[TILE<D>], ld[TILE<D>];
    __shared__ __attribute__((aligned(16))) float aux[4 * BS];
    const int lane = threadIdx.x;
    const int gq = lane >> 4, nq = lane & 15;
    const long kblk = xcd_block(blockIdx.x, gridDim.x);
    const int gh = (int)(kblk / g.n[1]), j = (int)(kblk % g.n[1]);
    const bool enrich1 = g.l0 == 1;  // level-1 pooled tokens enrich
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const long tbase = (long)gh * g.N;
    const long kbase = hbase + (long)j * BS * D;
    bf16x8 bk[NI], bv[NI];  // the key block's rows lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        bk[u] = ld8(k + kbase + nq * D + 32 * u + 8 * gq);
        bv[u] = ld8(v + kbase + nq * D + 32 * u + 8 * gq);
    }
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* list = w.col[0] + (long)gh * g.n[1] * g.K;
    const unsigned char* slots = w.slot[0] + (long)gh * g.n[1] * g.K;
    const int beg = uniform(rp[j]), end = uniform(rp[j + 1]);
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    f32x4 accK[ND] = {}, accV[ND] = {};
    // live == false (the padding step of an odd-length chunk): the MFMAs run
    // on valid rows but every P and dS is 0
    // per-row scalars as the step uses them: -lse * log2(e) (lanes < 16), so
    // that P = exp2(S c - lse log2 e) is one fma and one exp2; in the padding
    // step (live == false) -inf there and 0 for the pooled P and dS, which
    // makes every P and dS of the step exactly 0
    const bool lse_lane = lane < 16, pe_lane = lane >= 32;
    auto step = [&](const QBlock<D>& f, bool live) {
        put_rows<D>(lq, f.q, lane);
        put_rows<D>(ld, f.d, lane);
        const float nls = live ? -LOG2E * f.x : -INFINITY;
        aux[lane] = lse_lane ? nls : (pe_lane && !live) ? 0.f : f.x;
        lds_fence();
        const float4 l4 = *(const float4*)(aux + 4 * gq);
        const float4 e4 = *(const float4*)(aux + BS + 4 * gq);
        const float4 p4 = *(const float4*)(aux + 2 * BS + 4 * gq);
        const float4 s4 = *(const float4*)(aux + 3 * BS + 4 * gq);
        bf16x8 aq[NI], ad[NI];
        operand_rows<D, TS::ROW_T>(lq, aq, lane);
        operand_rows<D, TS::ROW_T>(ld, ad, lane);
        const f32x4 s = scores<D>(aq, bk);   // S[query][key]
        const f32x4 dp = scores<D>(ad, bv);  // dP[query][key]
        const float lr[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dr[4] = {e4.x, e4.y, e4.z, e4.w};
        const float pr[4] = {p4.x, p4.y, p4.z, p4.w};
        const float sr_[4] = {s4.x, s4.y, s4.z, s4.w};
        bf16x4 bp, bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float p = fast_exp2(fmaf(s[r], c, lr[r]));
            float ds = p * (dp[r] - dr[r]);
            if (enrich1) {
                p = fmaf(pr[r], 1.0f / BS, p);
                ds = fmaf(sr_[r], 1.0f / BS, ds);
            }
            bp[r] = (bf16)p;
            bs[r] = (bf16)ds;
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const int off = (4 * gq + rr) * TS::ROW_T + 16 * d + 4 * xx;
            accV[d] = mfma16(lds_read_tr(ld + off), bp, accV[d]);
            accK[d] = mfma16(lds_read_tr(lq + off), bs, accK[d]);
        }
    };
    // the list is read 64 entries at a time, one per lane, and each step takes
    // its query block and slot with readlane, so no load waits on another
    int myi = 0, mys = 0;
    // buffer loads: rows sr + RPI u of block i at lane offset voff + 1024 u,
    // block offset i * 32 D bytes; one dword per lane carries the block's
    // per-row scalars (lse, delta, pooled P and dS), each lane reading from
    // one of three resources -- the other two give 0 for an out-of-range
    // offset -- so there is no divergent branch
    const unsigned head_bytes = (unsigned)g.N * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + hbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dout + hbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rlse = make_rsrc(lse + tbase, (unsigned)g.N * 4);
    const __amdgpu_buffer_rsrc_t rdel = make_rsrc(w.delta + tbase, (unsigned)g.N * 4);
    const int sr = lane / TS::LPR, sc = (lane % TS::LPR) * 8;
    const int voff = (sr * D + sc) * 2;
    const int off_lse = lane < 16 ? 4 * lane : OFF_NONE;
    const int off_del = (lane >= 16 && lane < 32) ? 4 * (lane - 16) : OFF_NONE;
    const int off_pe = lane >= 32 ? 4 * (lane - 32) : OFF_NONE;
    auto fetch = [&](QBlock<D>& f, int t) {
        const int i = __builtin_amdgcn_readlane(myi, t);
        const int sl = __builtin_amdgcn_readlane(mys, t);
        const int so = i * (BS * D * 2);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.q[u] = bload8(rq, voff + 1024 * u, so);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.d[u] = bload8(rdo, voff + 1024 * u, so);
        const __amdgpu_buffer_rsrc_t rpe =
            make_rsrc(w.pe1 + (((long)gh * g.n[1] + i) * g.K + sl) * 2 * BS, 2 * BS * 4);
        f.x = bloadf(rlse, off_lse, i * BS * 4) + bloadf(rdel, off_del, i * BS * 4) +
              bloadf(rpe, off_pe, 0);
    };
    // two register sets alternate, each filled one step before it is used.
    // The loop body is one basic block: a conditional exit between a fetch
    // and its use would let the compiler sink the loads down to the use.
    // Fetches past the end re-read the last block (valid memory).
    QBlock<D> A, B;
    for (int cb = beg; cb < end; cb += 64) {
        const int n = min(64, end - cb);
        myi = lane < n ? list[cb + lane] : 0;
        mys = lane < n ? (int)slots[cb + lane] : 0;
        fetch(A, 0);
        for (int t = 0; t < n; t += 2) {
            fetch(B, min(t + 1, n - 1));
            step(A, true);
            fetch(A, min(t + 2, n - 1));
            step(B, t + 1 < n);
        }
    }
    // epilogue: scale, add the pooled-level gradients (levels >= 2), store
    const long obase = kbase + nq * D + 4 * gq;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
        float xk[4], xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xk[r] = accK[d][r] * g.scale;
            xv[r] = accV[d][r];
        }
        for (int l = max(2, g.l0); l <= g.L; ++l) {
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

// One wave per row, lane = channels lane + 64 c: every dot product is a wave
// sum.

// <a, row> over the D channels, a held as the lane's channels
template <int D>
__device__ __forceinline__ float row_dot(const float (&a)[D / 64], const float* row, int lane)
{
    float part = a[0] * row[lane];
#pragma unroll
    for (int c = 1; c < D / 64; ++c) part = fmaf(a[c], row[lane + 64 * c], part);
    return wave_sum(part);
}

template <int D>
__device__ __forceinline__ void lane_channels(float (&x)[D / 64], const float* row, int lane)
{
#pragma unroll
    for (int c = 0; c < D / 64; ++c) x[c] = row[lane + 64 * c];
}

template <int D, typename F>
__device__ __forceinline__ void for_each_entry(const Geo& g, const Ws& w, const float* k,
                                               const float* v, int gh, int t, F f)
{
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + t / BS) * g.K;
    for (int s = 0; s < g.K; ++s)
        for (int r = 0; r < BS; ++r) {
            long row = ((long)gh * g.N + (long)sel[s] * BS + r) * D;
            f(k + row, v + row, 0.f);
        }
    // enriching levels l0..L; a level-lv token's logit gets lb2 * lv * ln 2
    for (int lv = g.l0; lv <= g.L; ++lv) {
        const int a = t >> (4 * lv);
        const int* sl = w.idx[lv - 1] + ((long)gh * g.n[lv] + a) * g.Kl[lv];
        const float bias = g.lb2 * (float)lv * LN2;
        for (int s = 0; s < g.Kl[lv]; ++s) {
            long row = ((long)gh * g.n[lv] + sl[s]) * D;
            f(w.kbar[lv - 1] + row, w.vbar[lv - 1] + row, bias);
        }
    }
}

// dq and delta: one wave per query token
template <int D>
__global__ __launch_bounds__(256) void dq_f32(const float* __restrict__ q,
                                              const float* __restrict__ k,
                                              const float* __restrict__ v,
                                              const float* __restrict__ o,
                                              const float* __restrict__ lse,
                                              const float* __restrict__ dout,
                                              float* __restrict__ dq, Geo g, Ws w)
{
    constexpr int NC = D / 64;
    const long tg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (tg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    float qc[NC], dc[NC], acc[NC];
    lane_channels<D>(qc, q + tg * D, lane);
    lane_channels<D>(dc, dout + tg * D, lane);
    const float Dt = row_dot<D>(dc, o + tg * D, lane);
    if (lane == 0) w.delta[tg] = Dt;
    const float lt = lse[tg];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.f;
    for_each_entry<D>(g, w, k, v, gh, t, [&](const float* kr, const float* vr, float bias) {
        float kc[NC];
        lane_channels<D>(kc, kr, lane);
        const float z = row_dot<D>(qc, kr, lane);
        const float dp = row_dot<D>(dc, vr, lane);
        const float P = expf(z * g.scale + bias - lt);
        const float ds = P * (dp - Dt) * g.scale;
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = fmaf(ds, kc[c], acc[c]);
    });
#pragma unroll
    for (int c = 0; c < NC; ++c) dq[tg * D + lane + 64 * c] = acc[c];
}

// pooled-token gradients, every level: one wave per level-l block
template <int D>
__global__ __launch_bounds__(256) void enrich_f32(const float* __restrict__ q,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ dout, Geo g, Ws w,
                                                  int l)
{
    constexpr int NC = D / 64;
    const long blk = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (blk >= (long)g.G * g.n[l]) return;
    const int lane = threadIdx.x & 63;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    float kb[NC], vb[NC], sk[NC], sv[NC];
    lane_channels<D>(kb, w.kbar[l - 1] + blk * D, lane);
    lane_channels<D>(vb, w.vbar[l - 1] + blk * D, lane);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * g.Kl[l];
    const long span = 1l << (4 * l);
    const float bias = g.lb2 * (float)l * LN2;  // size bias of a level-l token
#pragma unroll
    for (int c = 0; c < NC; ++c) sk[c] = sv[c] = 0.f;
    for (int e = rp[j]; e < rp[j + 1]; ++e) {
        const long a = cl[e];
        for (long t = a * span; t < (a + 1) * span; ++t) {
            const long tg = (long)gh * g.N + t;
            float qc[NC], dc[NC];
            lane_channels<D>(qc, q + tg * D, lane);
            lane_channels<D>(dc, dout + tg * D, lane);
            const float z = row_dot<D>(kb, q + tg * D, lane);
            const float dp = row_dot<D>(vb, dout + tg * D, lane);
            const float P = expf(z * g.scale + bias - lse[tg]);
            const float ds = P * (dp - w.delta[tg]);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                sk[c] = fmaf(ds * g.scale, qc[c], sk[c]);
                sv[c] = fmaf(P, dc[c], sv[c]);
            }
        }
    }
    float* dst = w.dbar[l - 1] + blk * 2 * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        dst[lane + 64 * c] = sk[c];
        dst[D + lane + 64 * c] = sv[c];
    }
}

// dk, dv: one wave per key token
template <int D>
__global__ __launch_bounds__(256) void dkdv_f32(const float* __restrict__ q,
                                                const float* __restrict__ k,
                                                const float* __restrict__ v,
                                                const float* __restrict__ lse,
                                                const float* __restrict__ dout,
                                                float* __restrict__ dk, float* __restrict__ dv,
                                                Geo g, Ws w)
{
    constexpr int NC = D / 64;
    const long xg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (xg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63;
    const int gh = (int)(xg / g.N), x = (int)(xg % g.N), j = x / BS;
    float kc[NC], vc[NC], ak[NC], av[NC];
    lane_channels<D>(kc, k + xg * D, lane);
    lane_channels<D>(vc, v + xg * D, lane);
#pragma unroll
    for (int c = 0; c < NC; ++c) ak[c] = av[c] = 0.f;
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* cl = w.col[0] + (long)gh * g.n[1] * g.K;
    for (int e = rp[j]; e < rp[j + 1]; ++e)
        for (int r = 0; r < BS; ++r) {
            const long tg = (long)gh * g.N + (long)cl[e] * BS + r;
            float qc[NC], dc[NC];
            lane_channels<D>(qc, q + tg * D, lane);
            lane_channels<D>(dc, dout + tg * D, lane);
            const float z = row_dot<D>(kc, q + tg * D, lane);
            const float dp = row_dot<D>(vc, dout + tg * D, lane);
            const float P = expf(z * g.scale - lse[tg]);
            const float ds = P * (dp - w.delta[tg]) * g.scale;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                ak[c] = fmaf(ds, qc[c], ak[c]);
                av[c] = fmaf(P, dc[c], av[c]);
            }
        }
    for (int l = g.l0; l <= g.L; ++l) {
        const float wgt = 1.0f / (float)(1 << (4 * l));
        const float* db = w.dbar[l - 1] + ((long)gh * g.n[l] + (x >> (4 * l))) * 2 * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            ak[c] += db[lane + 64 * c] * wgt;
            av[c] += db[D + lane + 64 * c] * wgt;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        dk[xg * D + lane + 64 * c] = ak[c];
        dv[xg * D + lane + 64 * c] = av[c];
    }
}

template <int D>
hipError_t launch_attn_dq_d(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, void* dq, int dtype,
                            const Geo& g, const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        auto kern = (g.n_pooled() <= 64) ? dq_bf16<64, D> : dq_bf16<MAX_E, D>;
        hipLaunchKernelGGL(kern, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, (const unsigned short*)out, lse,
                           (const unsigned short*)dout, (unsigned short*)dq, g, w);
    } else {
        long ntok = (long)g.G * g.N;  // one wave each
        hipLaunchKernelGGL(dq_f32<D>, dim3((unsigned)((ntok + 3) / 4)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, (const float*)out,
                           lse, (const float*)dout, (float*)dq, g, w);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_attn_dq_tr_d(const void* q, const void* k, const void* v, const void* out,
                               const float* lse, const void* dout, void* dq, const Geo& g,
                               const Ws& w, hipStream_t st)
{
    if (D == D128 || g.n_pooled() > 64) {
        // two launches at d = 128: there only two workgroups fit a CU, and the
        // transpose's long, mostly idle workgroups would hold dQ's slots (and
        // the large-entry variant has no registers to spare)
        hipError_t e = launch_transpose(g, w, st);
        if (e != hipSuccess) return e;
        return launch_attn_dq_d<D>(q, k, v, out, lse, dout, dq, LLSA_BF16, g, w, st);
    }
    const TrFirst tr = transpose_first(g);
    const int tr_pad = (tr.wgs + 7) & ~7;
    const long nblk = (long)g.G * g.n[1];
    hipLaunchKernelGGL((dq_tr_bf16<64, D>), dim3((unsigned)(tr_pad + (nblk + 3) / 4)), dim3(256), 0, st,
                       (const unsigned short*)q, (const unsigned short*)k,
                       (const unsigned short*)v, (const unsigned short*)out, lse,
                       (const unsigned short*)dout, (unsigned short*)dq, g, w, tr, tr_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_transpose_after(g, w, tr, st);
}

template <int D>
hipError_t launch_attn_enrich_d(const void* q, const float* lse, const void* dout, int dtype,
                                const Geo& g, const Ws& w, hipStream_t st)
{
    if (g.l0 > g.L) return hipSuccess;
    if (dtype == LLSA_BF16) {
        if (g.L < 2) return hipSuccess;
        hipLaunchKernelGGL(enrich_bwd_bf16<D>, dim3(g.G * g.n[2]), dim3(256), 0, st,
                           (const unsigned short*)q, lse, (const unsigned short*)dout, g, w);
        hipError_t e = hipGetLastError();
        for (int l = 2; l <= g.L && e == hipSuccess; ++l) {
            long n = (long)g.G * g.n[l];
            hipLaunchKernelGGL(enrich_sum<D>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, g,
                               w, l);
            e = hipGetLastError();
        }
        return e;
    }
    hipError_t e = hipSuccess;
    for (int l = g.l0; l <= g.L && e == hipSuccess; ++l) {
        long n = (long)g.G * g.n[l];  // one wave per pooled block
        hipLaunchKernelGGL(enrich_f32<D>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st,
                           (const float*)q, lse, (const float*)dout, g, w, l);
        e = hipGetLastError();
    }
    return e;
}

template <int D>
hipError_t launch_attn_dkdv_d(const void* q, const void* k, const void* v, const float* lse,
                              const void* dout, void* dk, void* dv, int dtype, const Geo& g,
                              const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        hipLaunchKernelGGL(dkdv_bf16<D>, dim3((unsigned)nblk), dim3(64), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, lse, (const unsigned short*)dout,
                           (unsigned short*)dk, (unsigned short*)dv, g, w);
    } else {
        long ntok = (long)g.G * g.N;  // one wave per key token
        hipLaunchKernelGGL(dkdv_f32<D>, dim3((unsigned)((ntok + 3) / 4)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, lse,
                           (const float*)dout, (float*)dk, (float*)dv, g, w);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_dq(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, int dtype, const Geo& g,
                          const Ws& w, hipStream_t st)
{
    return g.d == D128 ? launch_attn_dq_d<D128>(q, k, v, out, lse, dout, dq, dtype, g, w, st)
                       : launch_attn_dq_d<D64>(q, k, v, out, lse, dout, dq, dtype, g, w, st);
}

hipError_t launch_attn_dq_transpose(const void* q, const void* k, const void* v, const void* out,
                                    const float* lse, const void* dout, void* dq, const Geo& g,
                                    const Ws& w, hipStream_t st)
{
    return g.d == D128 ? launch_attn_dq_tr_d<D128>(q, k, v, out, lse, dout, dq, g, w, st)
                       : launch_attn_dq_tr_d<D64>(q, k, v, out, lse, dout, dq, g, w, st);
}

// Gradients of the enriching pooled tokens (bf16: levels >= 2, level 1 being
// handled in the dk/dv pass; fp32: every enriching level).  Needs delta from
// the dq pass.
hipError_t launch_attn_enrich(const void* q, const float* lse, const void* dout, int dtype,
                              const Geo& g, const Ws& w, hipStream_t st)
{
    return g.d == D128 ? launch_attn_enrich_d<D128>(q, lse, dout, dtype, g, w, st)
                       : launch_attn_enrich_d<D64>(q, lse, dout, dtype, g, w, st);
}

hipError_t launch_attn_dkdv(const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, void* dk, void* dv, int dtype, const Geo& g,
                            const Ws& w, hipStream_t st)
{
    return g.d == D128 ? launch_attn_dkdv_d<D128>(q, k, v, lse, dout, dk, dv, dtype, g, w, st)
                       : launch_attn_dkdv_d<D64>(q, k, v, lse, dout, dk, dv, dtype, g, w, st);
}

}  // namespace llsa
