// k_attn_fwd.hip -- sparse attention forward with hierarchical KV enrichment.
//
// LLSA README, usage: a drop-in for non-causal scaled-dot-product attention;
// skill summary, "Core Technique" 2: the key/value set of a query is enriched
// with coarse (pooled) tokens from several hierarchy levels.
//
// Key/value set of the 16 tokens of query block i (level-l ancestor
// a_l = i / 16^(l-1)):
//   - the 16*K tokens of the key blocks idx_1[i] (fine tiles, 16 keys each);
//   - for every enriching level l = l0..L the pooled pairs (kbar_l[j],
//     vbar_l[j]) for j in idx_l[a_l]; l0 = 1 by default, 2 with
//     LLSA_ENRICH_COARSE, none with LLSA_NO_ENRICH.
// One softmax over the whole set, scale 1/sqrt(d); lse in natural log.  With
// LLSA_SIZE_BIAS a level-l pooled logit gets + ln 16^l, as if the token stood
// for its 16^l keys.
//
// The pooled entries of the enriching levels (the sum of their top-k) form
// extra tiles of 16, read from the bf16 copy of the pyramid that the pool
// pass writes.
//
// bf16 kernels (MFMA): attn_fwd_u4 (below; K <= 16) gives a wave four
// sibling query blocks and loads each tile they share once;
// attn_fwd_bf16 (any K) gives a wave one query block:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, A = key rows, B = query rows;
//                    lane (g = lane/16, n = lane%16) holds S^T[4g + r][n]:
//                    four keys of query n, so softmax statistics of query n
//                    are reduced over lanes n, n+16, n+32, n+48 only.
//   O^T += V^T P^T   A = V^T from LDS with ds_read_b64_tr_b16 (values are
//                    staged row-major, read back transposed), B = P^T taken
//                    straight from the S^T accumulator layout: two 16-key
//                    tiles form the 32-deep contraction.
// fp32 kernel (VALU): one wave per query token (lane = channel), explicit
// pooled tokens.
#include "common.h"

namespace llsa {
namespace {

// Staged 16-row tiles in LDS (TileShape<D>): rows read back transposed
// (ds_read_b64_tr_b16, 4 rows x 32 B per 16 lanes) use a stride of D + 16
// elements, rows read as MFMA operands (ds_read_b128) D + 8; both spread their
// accesses over all banks.

__device__ __forceinline__ bf16x8 ld_bf16x8(const unsigned short* p)
{
    return *(const bf16x8*)p;
}

// Registers of one prefetched pair of fine tiles: load u of a tile holds row
// vr + RPI u (vr = lane / LPR), columns vc .. vc + 7 (vc = 8 (lane % LPR)) of
// the key and value tiles a and b.  Every load instruction covers whole rows,
// 1024 bytes, the fast gather pattern of the vector L1.
template <int D>
struct FinePair {
    static constexpr int NI = TileShape<D>::NI;
    bf16x8 ka[NI], kb[NI], va[NI], vb[NI];
};

// A operand of S^T = K Q^T from a staged key tile: row lane%16, channels
// 32u + 8(lane/16) .. +7 for u < D/32.
template <int D>
__device__ __forceinline__ void key_operand(const unsigned short* lds,
                                            bf16x8 (&k)[TileShape<D>::NI], int lane)
{
    operand_rows<D, TileShape<D>::ROW_A>(lds, k, lane);
}

// Softmax state.  The exponentials use a reference max m that is raised only
// when a new logit exceeds it by more than TAU (log2 units), so P <= 2^TAU and
// the accumulators are rarely rescaled; the result is the same softmax.
constexpr float TAU = 8.0f;

template <int D>
struct Online {
    f32x4 acc[D / 16];  // O^T tiles: lane holds O^T[16d + 4(lane/16) + r][query lane%16]
    f32x4 den;          // softmax denominator of query lane%16 (all four equal): the
                        // same MFMA as O^T with an all-ones value tile, so it sums
                        // exactly the bf16 weights that multiply the values
    float m;            // reference max (log2 units), equal in the 4 lanes of a query
};

// One step over two 16-entry tiles whose values are staged in LDS at la / lb.
// na / nb: valid entries (MASK == false: both tiles full).
// MASK == true (the masked tail): entries of tile a at or past na (b: nb)
// are masked, and ba / bb add a logit bias to rows 4(lane/16) + r (log2
// units; pooled tokens under the size-weighted variant).
template <bool MASK, int D>
__device__ __forceinline__ void attend_pair(Online<D>& st, const bf16x8 (&bq)[TileShape<D>::NI],
                                            const bf16x8 (&ka)[TileShape<D>::NI],
                                            const bf16x8 (&kb)[TileShape<D>::NI],
                                            const unsigned short* la, const unsigned short* lb,
                                            int na, int nb, float c, int lane,
                                            const float* ba = nullptr, const float* bb = nullptr)
{
    const int gq = lane >> 4;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 sa = scores<D>(ka, bq);
    const f32x4 sb = scores<D>(kb, bq);
    float ya[4], yb[4];  // logits in log2 units, masked entries at -inf
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        ya[r] = (!MASK || 4 * gq + r < na) ? (MASK ? fmaf(sa[r], c, ba[r]) : sa[r] * c) : -INFINITY;
        yb[r] = (!MASK || 4 * gq + r < nb) ? (MASK ? fmaf(sb[r], c, bb[r]) : sb[r] * c) : -INFINITY;
    }
    // this lane's max; the 4-lane reduction is only needed when the
    // reference max must move (rarely, after the first pair)
    const float lm = fmaxf(fmaxf(fmaxf(ya[0], ya[1]), fmaxf(ya[2], ya[3])),
                           fmaxf(fmaxf(yb[0], yb[1]), fmaxf(yb[2], yb[3])));
    if (__ballot(lm > st.m + TAU)) {
        const float mnew = fmaxf(st.m, max_x4(lm));
        const float alpha = fast_exp2(st.m - mnew);
#pragma unroll
        for (int d = 0; d < D / 16; ++d) st.acc[d] *= alpha;
        st.den *= alpha;
        st.m = mnew;
    }
    bf16x8 pp;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pp[r] = (bf16)fast_exp2(ya[r] - st.m);
        pp[4 + r] = (bf16)fast_exp2(yb[r] - st.m);
    }
    lds_fence();
#pragma unroll
    for (int d = 0; d < D / 16; ++d) {
        const int off = (4 * gq + rr) * TileShape<D>::ROW_T + 16 * d + 4 * xx;
        bf16x4 va = lds_read_tr(la + off), vb = lds_read_tr(lb + off);
        bf16x8 av = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
        st.acc[d] = mfma32(av, pp, st.acc[d]);
    }
    const bf16 one = (bf16)1.0f;
    const bf16x8 ones = {one, one, one, one, one, one, one, one};
    st.den = mfma32(ones, pp, st.den);
}

constexpr int MAX_E = MAX_L * 64;  // pooled entries per query block (L * K)

// Per-wave LDS: two value tiles (160-byte rows), two key tiles (144-byte
// rows) and the table of pooled-entry rows (ECAP ints).  With ECAP = 64 a
// workgroup of 4 waves needs under 40 KB, so 4 workgroups share a CU.
template <int ECAP, int D>
struct FwdLds {
    static constexpr int V_TILE = BS * TileShape<D>::ROW_T;  // bf16 elements
    static constexpr int K_TILE = BS * TileShape<D>::ROW_A;
    static constexpr int PER_WAVE = 2 * V_TILE + 2 * K_TILE + 2 * ECAP;  // in bf16 units
};

template <int ECAP, int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16(const unsigned short* __restrict__ q,
                                                     const unsigned short* __restrict__ k,
                                                     const unsigned short* __restrict__ v,
                                                     unsigned short* __restrict__ out,
                                                     float* __restrict__ lse, Geo g, Ws w)
{
    using Lay = FwdLds<ECAP, D>;
    using TS = TileShape<D>;
    constexpr int NI = TS::NI;
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][Lay::PER_WAVE];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)xcd_block(blockIdx.x, gridDim.x) * 4 + wv;  // over G * n1
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const float c = g.scale * LOG2E;  // logits in log2 units
    const long hbase = (long)gh * g.N * D;
    const long qbase = hbase + (long)i * BS * D;
    bf16x8 bq[NI];  // B operand of S^T: query row lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
    for (int u = 0; u < NI; ++u) bq[u] = ld_bf16x8(q + qbase + nq * D + 32 * u + 8 * gq);
    // the query block's K fine blocks, one per lane (K <= 64)
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i) * g.K;
    const int myj = lane < g.K ? clampi(sel[lane], g.n[1]) : 0;
    // pooled entries e = eoff[l] + slot of the enriching levels l0..L: their
    // rows in the bf16 pooled arrays
    const int E = g.n_pooled();
    int* ent = (int*)(smem[wv] + 2 * Lay::V_TILE + 2 * Lay::K_TILE);
    for (int l = g.l0; l <= g.L; ++l) {
        const int Kl = g.Kl[l];
        const long a = (long)gh * g.n[l] + (i >> (4 * (l - 1)));
        for (int s0 = 0; s0 < Kl; s0 += 64)
            if (s0 + lane < Kl)
                ent[g.eoff[l] + s0 + lane] =
                    (int)(w.prow[l - 1] + (long)gh * g.n[l] +
                          clampi(w.idx[l - 1][a * Kl + s0 + lane], g.n[l]));
    }
    lds_fence();

    Online<D> st;
#pragma unroll
    for (int d = 0; d < D / 16; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.den = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    unsigned short* la = smem[wv];  // value tiles (transposed reads)
    unsigned short* lb = la + Lay::V_TILE;
    unsigned short* lka = lb + Lay::V_TILE;  // key tiles (operand reads)
    unsigned short* lkb = lka + Lay::K_TILE;

    // Fine tiles first: K/2 full pairs in a loop whose body is one basic
    // block (prefetch of the next pair, then this pair), so the compiler
    // keeps every load a full step ahead of its use.  Buffer loads: lane
    // offset of row vr (row vr + RPI u is 1024 u bytes on), tile offset
    // j * 32 D.  Then the masked tail: a lone fine tile (K odd) and the
    // pooled tiles.
    const int vr = lane / TS::LPR, vc = (lane % TS::LPR) * 8;
    const unsigned head_bytes = (unsigned)g.N * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + hbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + hbase, head_bytes);
    const int voff = (vr * D + vc) * 2;
    const int NF = g.K / 2;  // full fine pairs
    auto load_fine = [&](FinePair<D>& f, int p) {
        const int sa = __builtin_amdgcn_readlane(myj, 2 * p) * (BS * D * 2);
        const int sb = __builtin_amdgcn_readlane(myj, 2 * p + 1) * (BS * D * 2);
        // issue order: key rows, then value rows, of tile a, then of tile b
#pragma unroll
        for (int u = 0; u < NI; ++u) f.ka[u] = bload8(rk, voff + 1024 * u, sa);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.va[u] = bload8(rv, voff + 1024 * u, sa);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.kb[u] = bload8(rk, voff + 1024 * u, sb);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.vb[u] = bload8(rv, voff + 1024 * u, sb);
    };
    auto stage = [&](const FinePair<D>& f, bf16x8 (&ka)[NI], bf16x8 (&kb)[NI]) {
        stage_rows<D, TS::ROW_A>(lka, f.ka, lane);
        stage_rows<D, TS::ROW_A>(lkb, f.kb, lane);
        stage_rows<D, TS::ROW_T>(la, f.va, lane);
        stage_rows<D, TS::ROW_T>(lb, f.vb, lane);
        lds_fence();
        key_operand<D>(lka, ka, lane);
        key_operand<D>(lkb, kb, lane);
    };
    auto step_fine = [&](const FinePair<D>& f) {
        bf16x8 ka[NI], kb[NI];
        stage(f, ka, kb);
        attend_pair<false, D>(st, bq, ka, kb, la, lb, BS, BS, c, lane);
    };
    FinePair<D> A, B;
    if (NF > 0) {
        load_fine(A, 0);
        int p = 0;
        for (; p + 2 <= NF; p += 2) {
            load_fine(B, p + 1);
            step_fine(A);
            load_fine(A, min(p + 2, NF - 1));
            step_fine(B);
        }
        if (p < NF) step_fine(A);  // odd number of pairs: the last one is in A
    }
    // masked tail: tile t < NFT is the lone fine tile (K odd), then the
    // pooled tiles; pairs of tiles, rows read through per-lane pointers
    const int NFT = g.K & 1;
    const int NT = NFT + (E + BS - 1) / BS;
    const int jlast = __builtin_amdgcn_readlane(myj, g.K - 1);
    auto tail_off = [&](int t, int r) -> long {
        // element offset of row r (0..15) of tail tile t in k / v (the lone
        // fine tile) or in the pooled copies; rows past the last entry
        // repeat a valid one (they are masked)
        if (t < NFT) return hbase + ((long)jlast * BS + r) * D;
        return (long)ent[min(BS * (t - NFT) + r, E - 1)] * D;
    };
    for (int t = 0; t < NT; t += 2) {
        const int tb = min(t + 1, NT - 1);
        const bool fa = t < NFT, fb = tb < NFT;
        const unsigned short* kpa = fa ? k : w.kb16;
        const unsigned short* vpa = fa ? v : w.vb16;
        const unsigned short* kpb = fb ? k : w.kb16;
        const unsigned short* vpb = fb ? v : w.vb16;
        FinePair<D> f;
        long oa[NI], ob[NI];
#pragma unroll
        for (int u = 0; u < NI; ++u) {
            oa[u] = tail_off(t, vr + TS::RPI * u);
            ob[u] = tail_off(tb, vr + TS::RPI * u);
        }
#pragma unroll
        for (int u = 0; u < NI; ++u) f.ka[u] = ld_bf16x8(kpa + oa[u] + vc);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.va[u] = ld_bf16x8(vpa + oa[u] + vc);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.kb[u] = ld_bf16x8(kpb + ob[u] + vc);
#pragma unroll
        for (int u = 0; u < NI; ++u) f.vb[u] = ld_bf16x8(vpb + ob[u] + vc);
        bf16x8 ka[NI], kb[NI];
        stage(f, ka, kb);
        // valid entries of the two tiles, and each row's logit bias (that
        // of the level of pooled entry e)
        const int na = t < NFT ? BS : max(0, min(BS, E - BS * (t - NFT)));
        const int nb = t + 1 >= NT ? 0 : (t + 1 < NFT ? BS : max(0, min(BS, E - BS * (t + 1 - NFT))));
        float ba[4], bb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ea = BS * (t - NFT) + 4 * gq + r, eb = ea + BS;
            ba[r] = t < NFT ? 0.f : g.lb2 * (float)g.entry_level(ea);
            bb[r] = t + 1 < NFT ? 0.f : g.lb2 * (float)g.entry_level(eb);
        }
        attend_pair<true, D>(st, bq, ka, kb, la, lb, na, nb, c, lane, ba, bb);
    }

    const float lsum = st.den[0];
    const float inv = 1.0f / lsum;
    const long obase = qbase + nq * D + 4 * gq;
#pragma unroll
    for (int d = 0; d < D / 16; ++d) {
        u16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = f2bf(st.acc[d][r] * inv);
        *(u16x4*)(out + obase + 16 * d) = o;
    }
    if (gq == 0) lse[(long)gh * g.N + (long)i * BS + nq] = (st.m + fast_log2(lsum)) * LN2;
}

// --------------------------------------------- four sibling blocks per wave
//
// attn_fwd_u4 (every top-k <= 16): a wave owns four consecutive query blocks.  They
// are siblings (the same parent at every coarser level), so their fine picks
// overlap: the wave forms the ascending union of the 4 K picks (about 37 of
// 64 at 256x256, K = 16), loads every union tile once and applies it to each
// of its blocks that picked it.  The vector-memory traffic per unit of work
// drops by that overlap, and the four blocks' independent softmax chains
// give the wave more to issue while MFMA results are pending.  One 16-key
// tile per step: S^T = K Q^T (16x16x32 MFMA over the channels), then
// O^T += V^T P^T and the denominator with 16x16x16 MFMAs over the 16 keys.
// Pooled tiles follow: one level-1 tile per block (its picks' pooled rows),
// one tile per coarser level shared by all four (same ancestor).

// (d = 64 only: the four blocks' state fills the register file)
using TS64 = TileShape<D64>;

struct Tile {
    bf16x8 k[2], v[2];  // rows vr and vr+8, channels vc .. vc+7
};

struct Q4 {
    f32x4 acc[4];
    f32x4 den;
    float m;
};

// MASK == true: rows at or past na are masked and every logit gets the
// tile's bias b2 (log2 units; pooled tiles under the size-weighted variant)
template <bool MASK>
__device__ __forceinline__ void tile_step(Q4& st, bf16x8 bq0, bf16x8 bq1, bf16x8 ka0, bf16x8 ka1,
                                          const bf16x4 (&vt)[4], int na, float c, int lane,
                                          float b2 = 0.f)
{
    const int gq = lane >> 4;
    const f32x4 zero = {};
    const f32x4 sa = mfma32(ka1, bq1, mfma32(ka0, bq0, zero));
    float y[4];  // logits in log2 units, masked at -inf
#pragma unroll
    for (int r = 0; r < 4; ++r)
        y[r] = (!MASK || 4 * gq + r < na) ? (MASK ? fmaf(sa[r], c, b2) : sa[r] * c) : -INFINITY;
    const float lm = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
    if (__ballot(lm > st.m + TAU)) {
        const float mnew = fmaxf(st.m, max_x4(lm));
        const float alpha = fast_exp2(st.m - mnew);
#pragma unroll
        for (int d = 0; d < 4; ++d) st.acc[d] *= alpha;
        st.den *= alpha;
        st.m = mnew;
    }
    bf16x4 pp;
#pragma unroll
    for (int r = 0; r < 4; ++r) pp[r] = (bf16)fast_exp2(y[r] - st.m);
#pragma unroll
    for (int d = 0; d < 4; ++d) st.acc[d] = mfma16(vt[d], pp, st.acc[d]);
    const bf16 one = (bf16)1.0f;
    const bf16x4 ones = {one, one, one, one};
    st.den = mfma16(ones, pp, st.den);
}

constexpr int U4_PT = 4 + MAX_L - 1;  // pooled tiles per wave (4 level-1 + one per coarser level)

struct U4Lds {
    unsigned short k[BS * TS64::ROW_A];
    unsigned short v[BS * TS64::ROW_T];
    int arr[64];                  // the 4 x 16 picks (lane order), INT_MAX if unused
    int first[64];                // pick value if it is the first occurrence, else INT_MAX
    int tab[64];                  // union tile j
    int tmask[64];                // which of the 4 blocks picked it
    int pent[U4_PT * BS];         // pooled tile rows (row index into kb16 / vb16)
};

__global__ __launch_bounds__(256) void attn_fwd_u4(const unsigned short* __restrict__ q,
                                                   const unsigned short* __restrict__ k,
                                                   const unsigned short* __restrict__ v,
                                                   unsigned short* __restrict__ out,
                                                   float* __restrict__ lse, Geo g, Ws w)
{
    constexpr int D = D64;
    __shared__ __attribute__((aligned(16))) U4Lds sm[4];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const long qb0 = ((long)xcd_block(blockIdx.x, gridDim.x) * 4 + wv) * 4;  // over G * n1
    if (qb0 >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qb0 / g.n[1]), i0 = (int)(qb0 % g.n[1]);
    U4Lds& L = sm[wv];
    const float c = g.scale * LOG2E;
    const long hbase = (long)gh * g.N * D;
    const int K = g.K;
    const int E = g.n_pooled();

    // query operands of the four blocks
    bf16x8 bq0[4], bq1[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const long qb = hbase + ((long)(i0 + b) * BS + nq) * D + 8 * gq;
        bq0[b] = ld_bf16x8(q + qb);
        bq1[b] = ld_bf16x8(q + qb + 32);
    }
    // the 4 pick lists, lane 16 b + s holds pick s of block i0 + b
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i0) * K;
    const int my = (nq < K) ? clampi(sel[gq * K + nq], g.n[1]) : INT_MAX;
    L.arr[lane] = my;
    lds_fence();
    // union: first occurrences in lane order, their rank among distinct picks,
    // and the set of blocks that share each pick
    int dup = 0, mask = 0;
    for (int m = 0; m < 64; m += 4) {
        const int4 a4 = *(const int4*)&L.arr[m];
        const int av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool eq = av[t] == my;
            dup |= (eq && m + t < lane) ? 1 : 0;
            mask |= eq ? 1 << ((m + t) >> 4) : 0;
        }
    }
    const bool first = my != INT_MAX && !dup;
    L.first[lane] = first ? my : INT_MAX;
    lds_fence();
    int upos = 0;
    for (int m = 0; m < 64; m += 4) {
        const int4 f4 = *(const int4*)&L.first[m];
        upos += (f4.x < my) + (f4.y < my) + (f4.z < my) + (f4.w < my);
    }
    const int U = __popcll(__ballot(first));
    if (first) {
        L.tab[upos] = my;
        L.tmask[upos] = mask;
    }
    // pooled tile rows: when level 1 enriches, tiles 0..3 hold the level-1
    // pooled rows of blocks i0 + b's picks; then one tile per coarser level
    // l = 2..L (the common ancestor's picks)
    const int NT1 = (E && g.l0 == 1) ? 4 : 0;
    const int NPT = E ? NT1 + (g.L - max(g.l0, 2) + 1) : 0;
    auto tile_level = [&](int t) { return t < NT1 ? 1 : max(g.l0, 2) + (t - NT1); };
    if (E) {
        for (int t = 0; t < NPT; ++t) {
            if (lane < BS) {
                int row;
                if (t < NT1) {
                    row = (int)(w.prow[0] + (long)gh * g.n[1] + L.arr[t * 16 + min(lane, K - 1)]);
                } else {
                    const int l = tile_level(t), Kl = g.Kl[l];
                    const long a = (long)gh * g.n[l] + (i0 >> (4 * (l - 1)));
                    row = (int)(w.prow[l - 1] + (long)gh * g.n[l] +
                                clampi(w.idx[l - 1][a * Kl + min(lane, Kl - 1)], g.n[l]));
                }
                L.pent[t * BS + lane] = row;
            }
        }
    }
    lds_fence();
    const int tj = L.tab[lane], tm = L.tmask[lane];

    Q4 st[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int d = 0; d < 4; ++d) st[b].acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
        st[b].den = f32x4{0.f, 0.f, 0.f, 0.f};
        st[b].m = -INFINITY;
    }

    const int vr = lane >> 3, vc = (lane & 7) * 8;
    const unsigned head_bytes = (unsigned)g.N * D * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + hbase, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + hbase, head_bytes);
    const int voff = (vr * D + vc) * 2;
    auto load_union = [&](Tile& T, int u) {
        const int so = __builtin_amdgcn_readlane(tj, u) * (BS * D * 2);
        T.k[0] = bload8(rk, voff, so);
        T.k[1] = bload8(rk, voff + 8 * D * 2, so);
        T.v[0] = bload8(rv, voff, so);
        T.v[1] = bload8(rv, voff + 8 * D * 2, so);
    };
    auto load_pooled = [&](Tile& T, int t) {
        const long ra = (long)L.pent[t * BS + vr] * D + vc;
        const long rb = (long)L.pent[t * BS + vr + 8] * D + vc;
        T.k[0] = ld_bf16x8(w.kb16 + ra);
        T.k[1] = ld_bf16x8(w.kb16 + rb);
        T.v[0] = ld_bf16x8(w.vb16 + ra);
        T.v[1] = ld_bf16x8(w.vb16 + rb);
    };
    // stage a tile, then run it for the blocks in `members`
    auto run = [&](const Tile& T, int members, int na, auto masked, float b2 = 0.f) {
        stage_rows<D64, TS64::ROW_A>(L.k, T.k, lane);
        stage_rows<D64, TS64::ROW_T>(L.v, T.v, lane);
        lds_fence();
        bf16x8 ka[2];
        key_operand<D64>(L.k, ka, lane);
        bf16x4 vt[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            vt[d] = lds_read_tr(L.v + (4 * gq + rr) * TS64::ROW_T + 16 * d + 4 * xx);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if ((members >> b) & 1) {
                if (masked)
                    tile_step<true>(st[b], bq0[b], bq1[b], ka[0], ka[1], vt, na, c, lane, b2);
                else
                    tile_step<false>(st[b], bq0[b], bq1[b], ka[0], ka[1], vt, BS, c, lane);
            }
    };
    // union tiles, the next one in flight; the loop body has no conditional
    // exit between a load and its use.  A load past the end re-reads the
    // last tile (valid memory) and is not used.
    Tile A, B;
    if (U > 0) {
        load_union(A, 0);
        int u = 0;
        for (; u + 2 <= U; u += 2) {
            load_union(B, u + 1);
            run(A, __builtin_amdgcn_readlane(tm, u), BS, false);
            load_union(A, min(u + 2, U - 1));
            run(B, __builtin_amdgcn_readlane(tm, u + 1), BS, false);
        }
        if (u < U) run(A, __builtin_amdgcn_readlane(tm, u), BS, false);
    }
    if (NPT > 0) {
        // masked runs (rows at or past the tile level's K, logit bias of
        // the tile's level)
        auto members = [&](int t) { return t < NT1 ? 1 << t : 0xF; };
        auto bias = [&](int t) { return g.lb2 * (float)tile_level(t); };
        auto rows = [&](int t) { return g.Kl[tile_level(t)]; };
        load_pooled(A, 0);
        int t = 0;
        for (; t + 2 <= NPT; t += 2) {
            load_pooled(B, t + 1);
            run(A, members(t), rows(t), true, bias(t));
            load_pooled(A, min(t + 2, NPT - 1));
            run(B, members(t + 1), rows(t + 1), true, bias(t + 1));
        }
        if (t < NPT) run(A, members(t), rows(t), true, bias(t));
    }

#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float lsum = st[b].den[0];
        const float inv = 1.0f / lsum;
        const long obase = hbase + ((long)(i0 + b) * BS + nq) * D + 4 * gq;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            u16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = f2bf(st[b].acc[d][r] * inv);
            *(u16x4*)(out + obase + 16 * d) = o;
        }
        if (gq == 0)
            lse[(long)gh * g.N + (long)(i0 + b) * BS + nq] = (st[b].m + fast_log2(lsum)) * LN2;
    }
}

// ------------------------------------------------------------ fp32 path

// one wave per query token, lane = channels lane + 64 c: every logit is a
// wave sum
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse, Geo g, Ws w)
{
    constexpr int NC = D / 64;
    const long tg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (tg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    float qc[NC], o[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        qc[c] = q[tg * D + lane + 64 * c];
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    auto visit = [&](const float* kr, const float* vr, float bias) {
        float part = qc[0] * kr[lane];
#pragma unroll
        for (int c = 1; c < NC; ++c) part = fmaf(qc[c], kr[lane + 64 * c], part);
        const float z = wave_sum(part) * g.scale + bias;
        if (z > m) {
            const float a = expf(m - z);
            l *= a;
#pragma unroll
            for (int c = 0; c < NC; ++c) o[c] *= a;
            m = z;
        }
        const float p = expf(z - m);
        l += p;
#pragma unroll
        for (int c = 0; c < NC; ++c) o[c] = fmaf(p, vr[lane + 64 * c], o[c]);
    };
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + t / BS) * g.K;
    for (int s = 0; s < g.K; ++s)
        for (int r = 0; r < BS; ++r) {
            const long row = ((long)gh * g.N + (long)clampi(sel[s], g.n[1]) * BS + r) * D;
            visit(k + row, v + row, 0.f);
        }
    for (int lv = g.l0; lv <= g.L; ++lv) {  // pooled tokens of the enriching levels
        const int a = t >> (4 * lv);
        const int* sl = w.idx[lv - 1] + ((long)gh * g.n[lv] + a) * g.Kl[lv];
        const float bias = g.lb2 * (float)lv * LN2;
        for (int s = 0; s < g.Kl[lv]; ++s) {
            const long row = ((long)gh * g.n[lv] + clampi(sl[s], g.n[lv])) * D;
            visit(w.kbar[lv - 1] + row, w.vbar[lv - 1] + row, bias);
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) out[tg * D + lane + 64 * c] = o[c] / l;
    if (lane == 0) lse[tg] = m + logf(l);
}

template <int D>
hipError_t launch_attn_fwd_d(const void* q, const void* k, const void* v, void* out, float* lse,
                             int dtype, const Geo& g, const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        // the four-block kernel (d = 64): every fine list and every pooled
        // list fit one 16-entry tile
        bool fits = D == D64 && g.K <= BS && g.n[1] % 4 == 0;
        for (int l = g.l0; l <= g.L; ++l) fits = fits && g.Kl[l] <= BS;
        if (fits) {
            hipLaunchKernelGGL(attn_fwd_u4, dim3((unsigned)((nblk + 15) / 16)), dim3(256), 0, st,
                               (const unsigned short*)q, (const unsigned short*)k,
                               (const unsigned short*)v, (unsigned short*)out, lse, g, w);
        } else {
            auto kern = (g.n_pooled() <= 64) ? attn_fwd_bf16<64, D> : attn_fwd_bf16<MAX_E, D>;
            hipLaunchKernelGGL(kern, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
                               (const unsigned short*)q, (const unsigned short*)k,
                               (const unsigned short*)v, (unsigned short*)out, lse, g, w);
        }
    } else {
        long ntok = (long)g.G * g.N;  // one wave each
        hipLaunchKernelGGL(attn_fwd_f32<D>, dim3((unsigned)((ntok + 3) / 4)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, (float*)out, lse,
                           g, w);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                           int dtype, const Geo& g, const Ws& w, hipStream_t st)
{
    return g.d == D128 ? launch_attn_fwd_d<D128>(q, k, v, out, lse, dtype, g, w, st)
                       : launch_attn_fwd_d<D64>(q, k, v, out, lse, dtype, g, w, st);
}

}  // namespace llsa
