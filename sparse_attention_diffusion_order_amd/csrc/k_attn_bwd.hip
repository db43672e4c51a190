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
// LLSA_CAUSAL: the key/value set of the forward (the diagonal fine block
// masked to keys u <= t, no pooled token of an ancestor's own block, unused
// slots -1 skipped), so a key block's own query block sees it masked and does
// not count its level-1 pooled token.
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
// b) below K1 are level-1 pooled tokens; their P and dS are stored (bf16) at
// pe[entry][0 | 1][query] for the key-major dk/dv pass, which adds them at
// 1/16 weight to values it rounds to bf16 itself.
template <bool MASK, int D>
__device__ __forceinline__ void dq_pair(f32x4 (&acc)[D / 16], const bf16x8 (&bq)[D / 32],
                                        const bf16x8 (&bd)[D / 32], float nl2, float Dq,
                                        const bf16x8 (&ka)[D / 32], const bf16x8 (&kb)[D / 32],
                                        const bf16x8 (&va)[D / 32], const bf16x8 (&vb)[D / 32],
                                        const unsigned short* la, const unsigned short* lb,
                                        int na, int nb, float c, int lane, unsigned short* pe = nullptr,
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
                pe[e_a * 2 * BS + nq] = f2bf(Pa);
                pe[e_a * 2 * BS + BS + nq] = f2bf(dSa);
            }
            if (e_b < K1) {
                pe[e_b * 2 * BS + nq] = f2bf(Pb);
                pe[e_b * 2 * BS + BS + nq] = f2bf(dSb);
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
constexpr int CMP_E = 2048;        // the complement's entries per query block, at most

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
    const long qblk = (long)xcd_block(bid, nb, g.xcd_chunk) * 4 + wv;
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
    const int rawj = lane < g.K ? sel[lane] : -1;
    const int myj = lane < g.K ? clampi(rawj, g.n[1]) : 0;
    // fine tiles: K, or when causal the KF valid picks, the last of them the
    // diagonal tile; E1: the level-1 pooled entries (the picks but, when
    // causal, the block itself and the unused slots), at the picks' positions
    const int KF = g.causal ? max(1, (int)__popcll(__ballot(rawj >= 0))) : g.K;
    const int E1 = g.causal ? (int)__popcll(__ballot(rawj >= 0 && rawj != i)) : g.K;
    float Dq;
    {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            const bf16x8 ou = ld8_once(o + rowq + 32 * u + 8 * gq);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += (float)bd[u][e] * (float)ou[e];
        }
        Dq = sum_x4(s);
    }
    const long tok = (long)gh * g.N + (long)i * BS + nq;
    if (gq == 0) w.delta[tok] = Dq;
    const float nl2 = -lse[tok] * LOG2E;
    // the pooled entries of the enriching levels: rows in the bf16 pooled
    // arrays, with their level (fill_entries)
    int* ent = (int*)(smem[wv] + 2 * Lay::K_TILE + 2 * Lay::V_TILE);
    const int E = fill_entries(g, w, gh, i, ent, lane);
    lds_fence();

    f32x4 acc[D / 16] = {};
    unsigned short* la = smem[wv];  // key tiles
    unsigned short* lb = la + Lay::K_TILE;
    unsigned short* lva = lb + Lay::K_TILE;  // value tiles, read as operands only
    unsigned short* lvb = lva + Lay::V_TILE;
    // one pipeline over NF fine pairs then the pooled pairs, next pair in
    // flight; unconditional (clamped) loads keep the wait counts exact
    const int NF = (KF + 1) / 2;
    const int NFU = (g.causal ? KF - 1 : g.K) / 2;  // fine pairs without a mask
    const int NT = (E + BS - 1) / BS;
    const int NP = NF + (NT + 1) / 2;
    const int sr = lane / TS::LPR, sc = (lane % TS::LPR) * 8;
    auto load_pair = [&](DqPair<D>& f, int p) {
        long ka[NI], kb[NI];  // element offsets of row sr + RPI u of tiles a and b
        const unsigned short *kp, *vp;
        if (p < NF) {
            const int ja = __builtin_amdgcn_readlane(myj, min(2 * p, KF - 1));
            const int jb = __builtin_amdgcn_readlane(myj, min(2 * p + 1, KF - 1));
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
                ka[u] = (long)(ent[min(BS * t + sr + TS::RPI * u, E - 1)] & ENT_ROW) * D + sc;
                kb[u] = (long)(ent[min(BS * t + BS + sr + TS::RPI * u, E - 1)] & ENT_ROW) * D + sc;
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
    // SINGLE: one register set (d = 128, where two sets spill): the next
    // pair is loaded into it as soon as the current one is staged
    constexpr bool SINGLE = D == D128;
    auto step = [&](DqPair<D>& f, int p) {
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
        if (SINGLE) load_pair(f, min(p + 1, NP - 1));
        // full pairs of fine tiles run unmasked; with an odd count the last
        // fine "pair" holds the lone last tile twice (the clamped load), so
        // it takes the masked path with its second tile empty; the causal
        // diagonal tile (the last fine one) is masked to the keys at or
        // before each query row
        if (p < NFU) {
            dq_pair<false, D>(acc, bq, bd, nl2, Dq, ka, kb, va, vb, la, lb, BS, BS, c, lane);
        } else {
            auto fine_rows = [&](int t) {
                return t >= KF ? 0 : (g.causal && t == KF - 1) ? nq + 1 : BS;
            };
            const int e0 = p < NF ? 0 : BS * 2 * (p - NF);
            const int na = p < NF ? fine_rows(2 * p) : max(0, min(BS, E - e0));
            const int nb = p < NF ? fine_rows(2 * p + 1) : max(0, min(BS, E - e0 - BS));
            const bool pooled = p >= NF;
            // the level-1 picks' pooled entries (the first E1) keep their P
            // and dS for the key-major pass, at their picks' positions
            unsigned short* pe = (pooled && g.l0 == 1 && !g.cmp && e0 < E1)
                                     ? (unsigned short*)w.pe1 + ((long)gh * g.n[1] + i) * g.K * 2 * BS
                                     : nullptr;
            float ba[4], bb[4];  // pooled rows: the logit bias of the entry's level
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ea = e0 + 4 * gq + r;
                const bool bias = pooled && g.lb2 != 0.f;
                ba[r] = bias ? g.lb2 * (float)ent_level(ent[max(0, min(ea, E - 1))]) : 0.f;
                bb[r] = bias ? g.lb2 * (float)ent_level(ent[max(0, min(ea + BS, E - 1))]) : 0.f;
            }
            dq_pair<true, D>(acc, bq, bd, nl2, Dq, ka, kb, va, vb, la, lb, na, nb, c, lane, pe,
                             e0, E1, ba, bb);
        }
    };
    if (SINGLE) {
        DqPair<D> A;
        load_pair(A, 0);
        for (int p = 0; p < NP; ++p) step(A, p);
    } else {
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

// The pooled-token gradients of levels >= 2 over one level-2 block's 256
// query tokens.  The (level, 16-entry tile) pairs of the block's lists are
// taken NP at a time: each query block's Q and dO tiles are loaded once per
// NP pairs (NP = 2 at d = 64 when there are two or more pairs: with three
// levels the query rows are read once, not once per level).
template <int D, int NP>
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
    // query blocks past the last level-1 block (under a partial last level-2
    // block) do not exist: their rows are read from the last block instead
    // and their weights are 0
    auto row_addr = [&](int u) {
        const int i = min(16 * a2 + 4 * wv + u, g.n[1] - 1);
        return ((long)gh * g.N + (long)i * BS + sr) * D + sc;
    };
    auto load_rows = [&](bf16x8 (&xq)[NI], bf16x8 (&xd)[NI], long a) {
#pragma unroll
        for (int v = 0; v < NI; ++v) xq[v] = ld8(q + a + (long)TS::RPI * v * D);
#pragma unroll
        for (int v = 0; v < NI; ++v) xd[v] = ld8(dout + a + (long)TS::RPI * v * D);
    };
    {
        const int i = min(16 * a2 + 4 * wv + (lane >> 4), g.n[1] - 1);
        const long t0 = (long)gh * g.N + (long)i * BS + (lane & 15);
        rowst[wv][0][lane] = lse[t0];
        rowst[wv][1][lane] = w.delta[t0];
    }
    // the pairs: level l = 2..L, entry tiles e0 = 0, 16, .. below K_l
    int npairs = 0;
    for (int l = 2; l <= g.L; ++l) npairs += (g.Kl[l] + BS - 1) / BS;
    for (int p0 = 0; p0 < npairs; p0 += NP) {
        int lv[NP], e0[NP];
        bool on[NP];  // pair p0 + pp exists
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
            int p = min(p0 + pp, npairs - 1), l = 2;
            for (; l < g.L && p >= (g.Kl[l] + BS - 1) / BS; ++l) p -= (g.Kl[l] + BS - 1) / BS;
            lv[pp] = l;
            e0[pp] = BS * p;
            on[pp] = p0 + pp < npairs;
        }
        bool ev[NP];  // this lane's entry (e0 + nq) is live
        bf16x8 bk[NP][NI], bv[NP][NI];  // entry rows lane%16, channels 32u + 8(lane/16) ..
        float lb[NP];                   // size bias of the pair's level (log2)
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
            const int l = lv[pp], al = a2 >> (4 * (l - 2)), Kl = g.Kl[l];
            const int* sel = w.idx[l - 1] + ((long)gh * g.n[l] + al) * Kl;
            lb[pp] = g.lb2 * (float)l;
            // a live entry: causal rows skip unused slots (-1) and the
            // ancestor's own block (their partials are written as zeros)
            const int en = e0[pp] + nq;
            const int sj = en < Kl ? sel[en] : -1;
            ev[pp] = on[pp] && en < Kl && (!g.causal || (sj >= 0 && sj != al));
#pragma unroll
            for (int u = 0; u < NI; ++u) bk[pp][u] = bv[pp][u] = bf16x8{};
            if (ev[pp]) {
                long off = ((long)gh * g.n[l] + clampi(sj, g.n[l])) * D;
#pragma unroll
                for (int u = 0; u < NI; ++u) {
                    bk[pp][u] = ld8f(w.kbar[l - 1] + off + 32 * u + 8 * gq);
                    bv[pp][u] = ld8f(w.vbar[l - 1] + off + 32 * u + 8 * gq);
                }
            }
        }
        f32x4 ak[NP][ND] = {}, av[NP][ND] = {};
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
            const float4 l4 = *(const float4*)&rowst[wv][0][u * BS + 4 * gq];
            const float4 d4 = *(const float4*)&rowst[wv][1][u * BS + 4 * gq];
            const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {d4.x, d4.y, d4.z, d4.w};
            const bool live = 16 * a2 + 4 * wv + u < g.n[1];
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) {
                if (!on[pp]) continue;  // wave-uniform
                f32x4 s = scores<D>(aq, bk[pp]);  // S[query][entry]
                f32x4 dp = scores<D>(ad, bv[pp]);
                bf16x4 pP, pS;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float P = (ev[pp] && live) ? fast_exp2(s[r] * c - lr[r] * LOG2E + lb[pp]) : 0.f;
                    pP[r] = (bf16)P;
                    pS[r] = (bf16)(P * (dp[r] - dr[r]));
                }
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    const int off = (4 * gq + rr) * TS::ROW_T + 16 * d + 4 * xx;
                    ak[pp][d] = mfma16(lds_read_tr(lq + off), pS, ak[pp][d]);
                    av[pp][d] = mfma16(lds_read_tr(ld + off), pP, av[pp][d]);
                }
            }
        }
        // reduce the four waves in a fixed order, per pair dk then dv
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
            if (!on[pp]) continue;  // workgroup-uniform
            const int l = lv[pp], Kl = g.Kl[l];
            for (int kind = 0; kind < 2; ++kind) {
                __syncthreads();  // tiles (or the previous kind) no longer read
#pragma unroll
                for (int d = 0; d < ND; ++d)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[((wv * ND + d) * 4 + r) * 64 + lane] =
                            kind == 0 ? ak[pp][d][r] : av[pp][d][r];
                __syncthreads();
                for (int x = threadIdx.x; x < ND * 4 * 64; x += blockDim.x) {
                    const float s = red[x] + red[ND * 256 + x] + red[2 * ND * 256 + x] +
                                    red[3 * ND * 256 + x];
                    const int d = x >> 8, r = (x >> 6) & 3, ln = x & 63;
                    const int ent = e0[pp] + (ln & 15), dim = 16 * d + 4 * (ln >> 4) + r;
                    if (ent < Kl) {
                        float* dst = w.part[l - 1] +
                                     ((((long)gh * g.n[2] + a2) * Kl + ent) * 2 + kind) * D;
                        dst[dim] = kind == 0 ? s * g.scale : s;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// dbar_l[j] = sum over level-l query blocks a that chose j, and over the
// level-2 blocks under a, of the partial sums at j's slot in a's list.  One
// workgroup per pooled block, lane = channels lane + 64 c: the list's
// (entry, level-2 block) rows, in ascending entry order, are split into four
// contiguous quarters, each summed in order by one wave, and the four sums
// are added in wave order.
template <int D>
__global__ __launch_bounds__(256) void enrich_sum(Geo g, Ws w, int l)
{
    constexpr int NC = D / 64;  // channels dim + 64 c per lane
    __shared__ float wsum[4][2][D];
    const long blk = blockIdx.x;
    if (blk >= (long)g.G * g.n[l]) return;  // workgroup-uniform
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int dim = lane;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int Kl = g.Kl[l];
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * Kl;
    const unsigned char* sl = w.slot[l - 1] + (long)gh * g.n[l] * Kl;
    const int span = 1 << (4 * (l - 2));  // level-2 blocks per level-l block
    const float* part = w.part[l - 1] + (long)gh * g.n[2] * Kl * 2 * D + dim;
    float sk[NC] = {}, sv[NC] = {};
    const int tot = g.n[l] * Kl;  // list entries of the head
    const int beg = uniform(clampi(rp[j], tot + 1)), end = uniform(max(beg, clampi(rp[j + 1], tot + 1)));
    // this wave's rows: a contiguous quarter of the (entry, level-2 block)
    // rows, taken in batches of 64 entries (lane e holds entry e0 + e: the
    // row offset into the partials), eight loads in flight at a time
    const long nrow_all = (long)(end - beg) * span;
    const long q_lo = nrow_all * wv / 4, q_hi = nrow_all * (wv + 1) / 4;
    for (long qb = q_lo; qb < q_hi;) {
        const int e0 = beg + (int)(qb / span);  // the batch's first entry
        const int ne = min(64, end - e0);
        int off = 0;   // in rows of 2*D floats
        int blk2 = 0;  // the entry's first level-2 block
        if (lane < ne) {
            const int a = clampi(cl[e0 + lane], g.n[l]);
            blk2 = a * span;
            off = a * span * Kl + clampi(sl[e0 + lane], Kl);
        }
        // rows qb .. qe of this batch (row q: entry q / span, block q % span)
        const long qe = min(q_hi, (long)(e0 - beg + ne) * span);
        for (long q0 = qb; q0 < qe; q0 += 8) {
            float vk[8][NC], vv[8][NC];
            bool ok[8];  // level-2 blocks past the last one (partial level-l block) do not exist
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const long qq = min(q0 + u, qe - 1);
                const int e = (int)(qq / span) - (e0 - beg), a2 = (int)(qq % span);
                ok[u] = q0 + u < qe && __builtin_amdgcn_readlane(blk2, e) + a2 < g.n[2];
                const int a2c = ok[u] ? a2 : 0;
                const long o = ((long)__builtin_amdgcn_readlane(off, e) + (long)a2c * Kl) * 2 * D;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    vk[u][c] = part[o + 64 * c];
                    vv[u][c] = part[o + D + 64 * c];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (ok[u])
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        sk[c] += vk[u][c];
                        sv[c] += vv[u][c];
                    }
        }
        qb = qe;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        wsum[wv][0][dim + 64 * c] = sk[c];
        wsum[wv][1][dim + 64 * c] = sv[c];
    }
    __syncthreads();
    if (wv == 0) {
        float* dst = w.dbar[l - 1] + blk * 2 * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int x = dim + 64 * c;
            dst[x] = ((wsum[0][0][x] + wsum[1][0][x]) + wsum[2][0][x]) + wsum[3][0][x];
            dst[D + x] = ((wsum[0][1][x] + wsum[1][1][x]) + wsum[2][1][x]) + wsum[3][1][x];
        }
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
    bool diag;  // causal and the query block is the key block itself
};

// Waves per workgroup of the dk/dv pass: WPG consecutive (sibling) key
// blocks, one independent wave each (no barriers), share a CU and so its L1
// and the timing of their overlapping query-block fetches.
constexpr int DKDV_WPG = 1;

// CAUSAL: LLSA_CAUSAL (its own instance, so that the default one carries no
// mask code).  ENRICH1: level 1's pooled tokens enrich (a compile-time
// switch: as a run-time one the compiler branches around the pooled terms of
// every row, each branch waiting on all outstanding LDS reads).  At most 3
// waves per SIMD: the compiler then schedules for that occupancy (147
// registers at d = 64); left to fit 4 (114 registers) the kernel is slower
// (256x256: 214.7 against 204.1 us; 512x512: 861 against 804 us), as more key
// blocks in flight per XCD spread the query blocks they gather over its L2.
template <int D, int WPG, bool CAUSAL, bool ENRICH1>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(1, 3))) void dkdv_bf16(const unsigned short* __restrict__ q,
                                                      const unsigned short* __restrict__ k,
                                                      const unsigned short* __restrict__ v,
                                                      const float* __restrict__ lse,
                                                      const unsigned short* __restrict__ dout,
                                                      unsigned short* __restrict__ dk,
                                                      unsigned short* __restrict__ dv, Geo g,
                                                      Ws w)
{
    using TS = TileShape<D>;
    constexpr int NI = TS::NI, ND = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned short lqs[WPG][TILE<D>], lds_[WPG][TILE<D>];
    __shared__ __attribute__((aligned(16))) float auxs[WPG][4 * BS];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    unsigned short* lq = lqs[wv];
    unsigned short* ld = lds_[wv];
    float* aux = auxs[wv];
    const int gq = lane >> 4, nq = lane & 15;
    const long kblk = (long)xcd_block(blockIdx.x, gridDim.x, g.xcd_chunk) * WPG + wv;
    if (kblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(kblk / g.n[1]), j = (int)(kblk % g.n[1]);
    constexpr bool enrich1 = ENRICH1;  // level-1 picks' pooled tokens enrich
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const long tbase = (long)gh * g.N;
    const long kbase = hbase + (long)j * BS * D;
    bf16x8 bk[NI], bv[NI];  // the key block's rows lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        bk[u] = ld8_once(k + kbase + nq * D + 32 * u + 8 * gq);
        bv[u] = ld8_once(v + kbase + nq * D + 32 * u + 8 * gq);
    }
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* list = w.col[0] + (long)gh * g.n[1] * g.K;
    const unsigned char* slots = w.slot[0] + (long)gh * g.n[1] * g.K;
    const int tot = g.n[1] * g.K;  // list entries of the head
    const int beg = uniform(clampi(rp[j], tot + 1)), end = uniform(max(beg, clampi(rp[j + 1], tot + 1)));
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
            // the causal diagonal block: key nq is seen by queries at or after it
            if (CAUSAL && f.diag && nq > 4 * gq + r) p = 0.f;
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
    const int off_pe = lane >= 32 ? 2 * (lane - 32) : OFF_NONE;  // bf16 P (32..47), dS (48..63)
    auto fetch = [&](QBlock<D>& f, int t) {
        const int i = __builtin_amdgcn_readlane(myi, t);
        const int sl = __builtin_amdgcn_readlane(mys, t);
        const int so = i * (BS * D * 2);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.q[u] = bload8(rq, voff + 1024 * u, so);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.d[u] = bload8(rdo, voff + 1024 * u, so);
        // (the causal diagonal block does not see block j's pooled token:
        // an empty resource reads 0)
        f.diag = CAUSAL && i == j;
        const __amdgpu_buffer_rsrc_t rpe = make_rsrc(
            (const unsigned short*)w.pe1 + (((long)gh * g.n[1] + i) * g.K + sl) * 2 * BS,
            f.diag ? 0u : 2 * BS * 2);
        f.x = bloadf(rlse, off_lse, i * BS * 4) + bloadf(rdel, off_del, i * BS * 4) +
              bload_bf16(rpe, off_pe, 0);
    };
    // two register sets alternate, each filled one step before it is used.
    // The loop body is one basic block: a conditional exit between a fetch
    // and its use would let the compiler sink the loads down to the use.
    // Fetches past the end re-read the last block (valid memory).  The loop
    // takes the blocks in pairs; an odd count's last block, already in A,
    // takes one step after it.
    QBlock<D> A, B;
    for (int cb = beg; cb < end; cb += 64) {
        const int n = min(64, end - cb);
        myi = lane < n ? clampi(list[cb + lane], g.n[1]) : 0;
        mys = lane < n ? clampi(slots[cb + lane], g.K) : 0;
        fetch(A, 0);
        for (int t = 0; t + 1 < n; t += 2) {
            fetch(B, t + 1);
            step(A, true);
            fetch(A, min(t + 2, n - 1));
            step(B, true);
        }
        if (n & 1) step(A, true);
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
        // pooled-token gradients of levels >= 2 (every enriching level with
        // the complement, whose level-1 gradients also come from dbar)
        for (int l = g.cmp ? g.l0 : max(2, g.l0); l <= g.L; ++l) {
            const int a = j >> (4 * (l - 1));
            const float wgt = 1.0f / (float)g.tokens(l, a);  // the mean's share of each token
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

// ------------------------------------------- complement pooled-token gradients
//
// With LLSA_ENRICH_COMPLEMENT the pooled token j of level l is attended by
// the query blocks under every level-l block a whose candidates hold j and
// that did not pick it: every level-L block when l = L, below it the existing
// children of the level-(l+1) blocks that picked j's parent (that level's
// key->query list of the parent).  A workgroup takes 16 sibling pooled keys
// 16p .. 16p+15 (they share these attendees), its four waves split the query
// tiles (16 tokens each), and per tile
//   S = Q Kbar^T, dP = dO Vbar^T (16x16x32 MFMA), P = exp(s S + bias - lse)
//   with P = 0 in the columns of the keys the attendee picked,
//   dS = P (dP - D), dVbar^T += dO^T P, dKbar^T += Q^T dS (16x16x16 MFMA).
// The waves' sums are reduced in LDS in a fixed order.  At the coarsest level
// the attendees are split further into `chunks` workgroups per group, whose
// partial sums (in the level-1 pooled P/dS buffer, unused by this variant)
// cmp_sum adds in chunk order; otherwise the sums go straight to dbar.
template <int D>
__global__ __launch_bounds__(256) void cmp_grad_bf16(const unsigned short* __restrict__ q,
                                                     const float* __restrict__ lse,
                                                     const unsigned short* __restrict__ dout,
                                                     Geo g, Ws w, int l, int chunks)
{
    using TS = TileShape<D>;
    constexpr int NI = TS::NI, ND = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned short tiles[4][2][TILE<D>];
    __shared__ __attribute__((aligned(16))) float auxs[4][2 * BS];
    float* red = (float*)&tiles[0][0][0];  // the cross-wave sums, after the last tile
    static_assert(sizeof(tiles) >= 4 * ND * 4 * 64 * sizeof(float), "reduction buffer");
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const int nl = g.n[l], groups = (nl + BS - 1) / BS;
    const int bid = blockIdx.x;
    const int gh = bid / (groups * chunks), p = (bid / chunks) % groups, ck = bid % chunks;
    const float c = g.scale * LOG2E;
    const float lb = g.lb2 * (float)l;  // size bias of a level-l pooled token (log2)
    // the 16 pooled keys (rows past the level's last block: the last row,
    // their columns masked)
    const bool col_ok = BS * p + nq < nl;
    const long krow = w.prow[l - 1] + (long)gh * nl + min(BS * p + nq, nl - 1);
    bf16x8 bk[NI], bv[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        bk[u] = *(const bf16x8*)(w.kb16 + krow * D + 32 * u + 8 * gq);
        bv[u] = *(const bf16x8*)(w.vb16 + krow * D + 32 * u + 8 * gq);
    }
    // attendees of the group and their query tiles: tile z of the workgroup
    // is tile z % tpa of attendee z / tpa
    const int tpa = 1 << (4 * (l - 1));  // level-1 blocks under a level-l block
    int na, a0 = 0;
    const int* plist = nullptr;  // l < L: the parent level's key->query list of p
    if (l == g.L) {
        const int per = (nl + chunks - 1) / chunks;
        a0 = ck * per;
        na = max(0, min(per, nl - a0));
    } else {
        const int np = g.n[l + 1], kp = g.Kl[l + 1];
        const int* rp = w.rowptr[l] + (long)gh * (np + 1);
        const int tot = np * kp;
        const int b = clampi(rp[p], tot + 1), e = max(b, clampi(rp[p + 1], tot + 1));
        plist = w.col[l] + (long)gh * tot + b;
        na = BS * (e - b);
    }
    const int Kl = g.Kl[l];
    const int* Il = w.idx[l - 1] + (long)gh * nl * Kl;
    const long hbase = (long)gh * g.N * D;
    const unsigned head_bytes = (unsigned)g.N * D * 2;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + hbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dout + hbase, head_bytes);
    const int sr = lane / TS::LPR, scol = (lane % TS::LPR) * 8;
    const int voff = (sr * D + scol) * 2;
    unsigned short* lq = tiles[wv][0];
    unsigned short* ld = tiles[wv][1];
    float* aux = auxs[wv];
    f32x4 accK[ND] = {}, accV[ND] = {};
    const long ntile = (long)na * tpa;
    for (long z = wv; z < ntile; z += 4) {
        const int k = (int)(z / tpa), t = (int)(z % tpa);
        const int a = l == g.L ? a0 + k : BS * clampi(plist[k >> 4], g.n[l + 1]) + (k & 15);
        const int qb = a * tpa + t;  // the tile's level-1 query block
        if (a >= nl || qb >= g.n[1]) continue;  // no such child / block (partial parent)
        // the keys of the group this attendee picked (excluded)
        int first;
        const unsigned picked = hit_mask(Il + (long)clampi(a, nl) * Kl, Kl, p, &first);
        const bool live = col_ok && !((picked >> nq) & 1u);
        const int so = qb * (BS * D * 2);
        bf16x8 xq[NI], xd[NI];
#pragma unroll
        for (int u = 0; u < NI; ++u) xq[u] = bload8(rq, voff + 1024 * u, so);
#pragma unroll
        for (int u = 0; u < NI; ++u) xd[u] = bload8(rdo, voff + 1024 * u, so);
        const long trow = (long)gh * g.N + (long)qb * BS;
        const float rowv = lane < BS ? -LOG2E * lse[trow + lane]
                                     : lane < 2 * BS ? w.delta[trow + lane - BS] : 0.f;
        put_rows<D>(lq, xq, lane);
        put_rows<D>(ld, xd, lane);
        if (lane < 2 * BS) aux[lane] = rowv;
        lds_fence();
        const float4 l4 = *(const float4*)(aux + 4 * gq);
        const float4 e4 = *(const float4*)(aux + BS + 4 * gq);
        bf16x8 aq[NI], ad[NI];
        operand_rows<D, TS::ROW_T>(lq, aq, lane);
        operand_rows<D, TS::ROW_T>(ld, ad, lane);
        const f32x4 sc = scores<D>(aq, bk);   // S[query][key]
        const f32x4 dp = scores<D>(ad, bv);  // dP[query][key]
        const float lr[4] = {l4.x, l4.y, l4.z, l4.w}, dr[4] = {e4.x, e4.y, e4.z, e4.w};
        bf16x4 bp, bs;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = live ? fast_exp2(fmaf(sc[r], c, lr[r] + lb)) : 0.f;
            bp[r] = (bf16)pr;
            bs[r] = (bf16)(pr * (dp[r] - dr[r]));
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const int off = (4 * gq + rr) * TS::ROW_T + 16 * d + 4 * xx;
            accV[d] = mfma16(lds_read_tr(ld + off), bp, accV[d]);
            accK[d] = mfma16(lds_read_tr(lq + off), bs, accK[d]);
        }
        wave_lds_sync();  // this tile's LDS reads are done before the next writes
    }
    // the four waves' sums in a fixed order, dK then dV
    const int groups_all = g.G * groups;
    for (int kind = 0; kind < 2; ++kind) {
        __syncthreads();
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[((wv * ND + d) * 4 + r) * 64 + lane] = kind == 0 ? accK[d][r] : accV[d][r];
        __syncthreads();
        for (int x = threadIdx.x; x < ND * 4 * 64; x += blockDim.x) {
            const float sum = red[x] + red[ND * 256 + x] + red[2 * ND * 256 + x] +
                              red[3 * ND * 256 + x];
            const int d = x >> 8, r = (x >> 6) & 3, ln = x & 63;
            const int key = ln & 15, dim = 16 * d + 4 * (ln >> 4) + r;
            const float val = kind == 0 ? sum * g.scale : sum;
            if (chunks == 1) {
                if (BS * p + key < nl)
                    w.dbar[l - 1][(((long)gh * nl + BS * p + key) * 2 + kind) * D + dim] = val;
            } else {  // partial of chunk ck: [chunk][group][key][kind][dim]
                w.pe1[((((long)ck * groups_all + (long)gh * groups + p) * BS + key) * 2 + kind) *
                          D + dim] = val;
            }
        }
    }
}

// The coarsest level's complement gradients: the chunks' partial sums, added
// in chunk order.  One thread per (key, kind, channel).
template <int D>
__global__ __launch_bounds__(256) void cmp_sum(Geo g, Ws w, int chunks)
{
    const int l = g.L, nl = g.n[l], groups = (nl + BS - 1) / BS;
    const long groups_all = (long)g.G * groups;
    const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= groups_all * BS * 2 * D) return;
    const long gk = id / (2 * D);  // (head, group, key)
    const int rest = (int)(id % (2 * D));
    const long gg = gk / BS;
    const int key = (int)(gk % BS);
    const int gh = (int)(gg / groups), p = (int)(gg % groups);
    if (BS * p + key >= nl) return;
    float s = 0.f;
    for (int ck = 0; ck < chunks; ++ck) s += w.pe1[(((long)ck * groups_all + gg) * BS + key) * 2 * D + rest];
    w.dbar[l - 1][((long)gh * nl + BS * p + key) * 2 * D + rest] = s;
}

// Workgroups per group for the coarsest level's complement gradients: about
// 256 query tiles each, bounded by the partial buffer (the level-1 pooled
// P/dS array, G * n1 * K * 32 floats).
int cmp_chunks(const Geo& g, int D)
{
    const int nl = g.n[g.L], groups = (nl + BS - 1) / BS;
    const long tiles = (long)nl << (4 * (g.L - 1));
    long want = (tiles + 255) / 256;
    const long cap = ((long)g.G * g.n[1] * g.K * 2 * BS) / ((long)g.G * groups * BS * 2 * D);
    want = want < cap ? want : cap;
    want = want < nl ? want : nl;
    return want < 1 ? 1 : (int)want;
}

// ------------------------------------------------------------ fp32 path

// One wave per row (a query token, a key token, or a pooled token); the rows
// it meets are visited 16 at a time with lane = row r + 16 channel group
// (RowBatch and its helpers): dot products are CH = D/4 fmas and a sum over
// the four channel groups, and row-weighted sums are reduced over the 16
// rows once, at the end.

// a wave's per-lane partial sums of CH channels, reduced over the 16 rows,
// stored by lanes 0, 16, 32, 48 (each its channel group), times `scale`
template <int D>
__device__ __forceinline__ void store_slice(float* row, float (&x)[D / 4], int lane,
                                            float scale = 1.f)
{
    constexpr int CH = D / 4;
#pragma unroll
    for (int c = 0; c < CH; ++c) x[c] = row16_sum(x[c]) * scale;
    if ((lane & 15) == 0) {
        float4* dst = (float4*)(row + CH * (lane >> 4));
#pragma unroll
        for (int u = 0; u < CH / 4; ++u)
            dst[u] = float4{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
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
    constexpr int CH = D / 4;
    const long tg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (tg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63, r = lane & 15;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    float qc[CH], dc[CH], acc[CH];
    load_slice<D>(qc, q + tg * D, lane);
    load_slice<D>(dc, dout + tg * D, lane);
    load_slice<D>(acc, o + tg * D, lane);  // o, for delta
    const float Dt = slice_dot<D>(dc, acc);
    if (lane == 0) w.delta[tg] = Dt;
    const float lt = lse[tg];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = 0.f;
    auto run = [&](const RowBatch& bt) {
        float kx[CH], vx[CH];
        load_slice<D>(kx, bt.k, lane);
        load_slice<D>(vx, bt.v, lane);
        const float z = slice_dot<D>(qc, kx);
        const float dp = slice_dot<D>(dc, vx);
        const float P = r < bt.n ? expf(z * g.scale + bt.bias - lt) : 0.f;
        const float ds = P * (dp - Dt);
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = fmaf(ds, kx[c], acc[c]);
    };
    for_each_batch<D>(g, w, k, v, gh, t, lane, run);
    store_slice<D>(dq + tg * D, acc, lane, g.scale);
}

// The query tokens tok0 + r of a 16-row batch (rows at or past n repeat the
// last one): this lane's channel slice of row r's q and dO, and row r's lse
// and delta.
template <int D>
struct QRow {
    float q[D / 4], d[D / 4];
    float lse, delta;
};

template <int D>
__device__ __forceinline__ void load_qrow(QRow<D>& x, const float* q, const float* dout,
                                          const float* lse, const float* delta, long tok0,
                                          int n, int lane)
{
    const long t = tok0 + min(lane & 15, n - 1);
    load_slice<D>(x.q, q + t * D, lane);
    load_slice<D>(x.d, dout + t * D, lane);
    x.lse = lse[t];
    x.delta = delta[t];
}

// pooled-token gradients, every level: one workgroup per level-l block,
// its four waves taking contiguous quarters of the block's chooser list; the
// four sums are added in wave order
template <int D>
__global__ __launch_bounds__(256) void enrich_f32(const float* __restrict__ q,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ dout, Geo g, Ws w,
                                                  int l)
{
    constexpr int CH = D / 4;
    __shared__ float wsum[4][2][D];
    const long blk = blockIdx.x;
    if (blk >= (long)g.G * g.n[l]) return;  // workgroup-uniform
    const int lane = threadIdx.x & 63, r = lane & 15, wv = threadIdx.x >> 6;
    const int gh = (int)(blk / g.n[l]), j = (int)(blk % g.n[l]);
    float kb[CH], vb[CH], sk[CH], sv[CH];
    load_slice<D>(kb, w.kbar[l - 1] + blk * D, lane);
    load_slice<D>(vb, w.vbar[l - 1] + blk * D, lane);
    const int* rp = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    const int* cl = w.col[l - 1] + (long)gh * g.n[l] * g.Kl[l];
    const long span = 1l << (4 * l);
    const float bias = g.lb2 * (float)l * LN2;  // size bias of a level-l token
#pragma unroll
    for (int c = 0; c < CH; ++c) sk[c] = sv[c] = 0.f;
    // the level-l blocks whose tokens attend j: those that picked it (its
    // key->query list), or with the complement those among whose candidates
    // it is and that did not pick it -- every level-L block, below L the
    // children of the level-(l+1) blocks that picked j's parent
    const int tot = g.n[l] * g.Kl[l];
    int beg = clampi(rp[j], tot + 1), end = max(beg, clampi(rp[j + 1], tot + 1));
    const int* pl = nullptr;  // the parent level's key->query list of j's parent
    if (g.cmp) {
        if (l == g.L) {
            beg = 0;
            end = g.n[l];
        } else {
            const int np = g.n[l + 1], kp = g.Kl[l + 1], ptot = np * kp;
            const int* prp = w.rowptr[l] + (long)gh * (np + 1);
            const int pb = clampi(prp[j >> 4], ptot + 1);
            const int pe = max(pb, clampi(prp[(j >> 4) + 1], ptot + 1));
            pl = w.col[l] + (long)gh * ptot + pb;
            beg = 0;
            end = BS * (pe - pb);
        }
    }
    const int Kl = g.Kl[l];
    const int e_lo = beg + (int)((long)(end - beg) * wv / 4);
    const int e_hi = beg + (int)((long)(end - beg) * (wv + 1) / 4);
    for (int e = e_lo; e < e_hi; ++e) {
        long a;
        if (!g.cmp) {
            a = clampi(cl[e], g.n[l]);
            if (g.causal && a == j) continue;  // its own block's mean: not seen
        } else {
            a = l == g.L ? e : BS * clampi(pl[e >> 4], g.n[l + 1]) + (e & 15);
            if (a >= g.n[l]) continue;
            const int* sel = w.idx[l - 1] + ((long)gh * g.n[l] + a) * Kl;
            bool picked = false;
            for (int s = 0; s < Kl; ++s) picked = picked || sel[s] == j;
            if (picked) continue;
        }
        // the block's tokens (those before N), 16 at a time
        const long t1 = min((a + 1) * span, (long)g.N);
        for (long t0 = a * span; t0 < t1; t0 += BS) {
            const int n = (int)min((long)BS, t1 - t0);
            QRow<D> x;
            load_qrow<D>(x, q, dout, lse, w.delta, (long)gh * g.N + t0, n, lane);
            const float z = slice_dot<D>(kb, x.q);
            const float dp = slice_dot<D>(vb, x.d);
            const float P = r < n ? expf(z * g.scale + bias - x.lse) : 0.f;
            const float ds = P * (dp - x.delta);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                sk[c] = fmaf(ds, x.q[c], sk[c]);
                sv[c] = fmaf(P, x.d[c], sv[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        sk[c] = row16_sum(sk[c]) * g.scale;
        sv[c] = row16_sum(sv[c]);
    }
    if (r == 0)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            wsum[wv][0][CH * (lane >> 4) + c] = sk[c];
            wsum[wv][1][CH * (lane >> 4) + c] = sv[c];
        }
    __syncthreads();
    if (wv == 0) {
        float* dst = w.dbar[l - 1] + blk * 2 * D;
        for (int x = lane; x < 2 * D; x += 64) {
            const float* ws = &wsum[0][0][0] + x;  // kind x / D, element x % D
            dst[x] = ((ws[0] + ws[2 * D]) + ws[4 * D]) + ws[6 * D];
        }
    }
}

// dk, dv: one wave per key token, over the 16 rows of each query block of
// its block's list
template <int D>
__global__ __launch_bounds__(256) void dkdv_f32(const float* __restrict__ q,
                                                const float* __restrict__ k,
                                                const float* __restrict__ v,
                                                const float* __restrict__ lse,
                                                const float* __restrict__ dout,
                                                float* __restrict__ dk, float* __restrict__ dv,
                                                Geo g, Ws w)
{
    constexpr int CH = D / 4;
    const long xg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (xg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63, r = lane & 15;
    const int gh = (int)(xg / g.N), x = (int)(xg % g.N), j = x / BS;
    float kc[CH], vc[CH], ak[CH], av[CH];
    load_slice<D>(kc, k + xg * D, lane);
    load_slice<D>(vc, v + xg * D, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) ak[c] = av[c] = 0.f;
    const int* rp = w.rowptr[0] + (long)gh * (g.n[1] + 1);
    const int* cl = w.col[0] + (long)gh * g.n[1] * g.K;
    const int tot = g.n[1] * g.K;
    const int beg = clampi(rp[j], tot + 1), end = max(beg, clampi(rp[j + 1], tot + 1));
    for (int e = beg; e < end; ++e) {
        const int i = clampi(cl[e], g.n[1]);
        // the causal diagonal block: the queries at or after key x
        const int r0 = (g.causal && cl[e] == j) ? x % BS : 0;
        QRow<D> y;
        load_qrow<D>(y, q, dout, lse, w.delta, (long)gh * g.N + (long)i * BS, BS, lane);
        const float z = slice_dot<D>(kc, y.q);
        const float dp = slice_dot<D>(vc, y.d);
        const float P = r >= r0 ? expf(z * g.scale - y.lse) : 0.f;
        const float ds = P * (dp - y.delta);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            ak[c] = fmaf(ds, y.q[c], ak[c]);
            av[c] = fmaf(P, y.d[c], av[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        ak[c] = row16_sum(ak[c]) * g.scale;
        av[c] = row16_sum(av[c]);
    }
    // the pooled-level gradients: dbar_l of the block's level-l ancestor,
    // each token's share 1 / (its tokens)
    for (int l = g.l0; l <= g.L; ++l) {
        const float wgt = 1.0f / (float)g.tokens(l, x >> (4 * l));
        float db[CH], dbv[CH];
        const float* src = w.dbar[l - 1] + ((long)gh * g.n[l] + (x >> (4 * l))) * 2 * D;
        load_slice<D>(db, src, lane);
        load_slice<D>(dbv, src + D, lane);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            ak[c] += db[c] * wgt;
            av[c] += dbv[c] * wgt;
        }
    }
    if (r == 0) {
        float4* ok = (float4*)(dk + xg * D + CH * (lane >> 4));
        float4* ov = (float4*)(dv + xg * D + CH * (lane >> 4));
#pragma unroll
        for (int u = 0; u < CH / 4; ++u) {
            ok[u] = float4{ak[4 * u], ak[4 * u + 1], ak[4 * u + 2], ak[4 * u + 3]};
            ov[u] = float4{av[4 * u], av[4 * u + 1], av[4 * u + 2], av[4 * u + 3]};
        }
    }
}

template <int D>
hipError_t launch_attn_dq_d(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, void* dq, int dtype,
                            const Geo& g, const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        const int me = g.max_pooled();
        auto kern = me <= 64 ? dq_bf16<64, D> : me <= MAX_E ? dq_bf16<MAX_E, D> : dq_bf16<CMP_E, D>;
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
    if (D == D128 || g.max_pooled() > 64) {
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
    if (dtype == LLSA_BF16 && g.cmp) {  // the complement's pooled tokens, every enriching level
        hipError_t e = hipSuccess;
        for (int l = g.l0; l <= g.L && e == hipSuccess; ++l) {
            const int groups = (g.n[l] + BS - 1) / BS;
            const int chunks = l == g.L ? cmp_chunks(g, D) : 1;
            hipLaunchKernelGGL(cmp_grad_bf16<D>, dim3((unsigned)(g.G * groups * chunks)), dim3(256),
                               0, st, (const unsigned short*)q, lse, (const unsigned short*)dout, g,
                               w, l, chunks);
            e = hipGetLastError();
            if (e == hipSuccess && chunks > 1) {
                const long n = (long)g.G * groups * BS * 2 * D;
                hipLaunchKernelGGL(cmp_sum<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g,
                                   w, chunks);
                e = hipGetLastError();
            }
        }
        return e;
    }
    if (dtype == LLSA_BF16) {
        if (g.L < 2) return hipSuccess;
        int npairs = 0;  // (level, 16-entry tile) pairs of levels >= 2
        for (int l = 2; l <= g.L; ++l) npairs += (g.Kl[l] + BS - 1) / BS;
        // two pairs per pass at d = 64 (at d = 128 two pairs spill)
        auto kern = enrich_bwd_bf16<D, 1>;
        if constexpr (D == D64)
            if (npairs >= 2) kern = enrich_bwd_bf16<D, 2>;
        hipLaunchKernelGGL(kern, dim3(g.G * g.n[2]), dim3(256), 0, st, (const unsigned short*)q,
                           lse, (const unsigned short*)dout, g, w);
        hipError_t e = hipGetLastError();
        for (int l = 2; l <= g.L && e == hipSuccess; ++l) {
            long n = (long)g.G * g.n[l];  // one workgroup per pooled block
            hipLaunchKernelGGL(enrich_sum<D>, dim3((unsigned)n), dim3(256), 0, st, g, w, l);
            e = hipGetLastError();
        }
        return e;
    }
    hipError_t e = hipSuccess;
    for (int l = g.l0; l <= g.L && e == hipSuccess; ++l) {
        long n = (long)g.G * g.n[l];  // one workgroup per pooled block
        hipLaunchKernelGGL(enrich_f32<D>, dim3((unsigned)n), dim3(256), 0, st, (const float*)q,
                           lse, (const float*)dout, g, w, l);
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
        const bool e1 = g.l0 == 1 && !g.cmp;  // level-1 picks' pooled tokens enrich
        auto kern = g.causal ? (e1 ? dkdv_bf16<D, DKDV_WPG, true, true> : dkdv_bf16<D, DKDV_WPG, true, false>)
                             : (e1 ? dkdv_bf16<D, DKDV_WPG, false, true> : dkdv_bf16<D, DKDV_WPG, false, false>);
        hipLaunchKernelGGL(kern, dim3((unsigned)((nblk + DKDV_WPG - 1) / DKDV_WPG)),
                           dim3(64 * DKDV_WPG), 0, st,
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
