// attn_block.h -- the sparse attention forward of one query block by one
// wave (bf16, MFMA): the body of the forward's one-block kernel
// (k_attn_fwd.hip), callable from any launch that owns a wave's LDS.
//
// LLSA README, usage: a drop-in for non-causal scaled-dot-product attention;
// skill summary, "Core Technique" 2: the key/value set of a query is enriched
// with coarse (pooled) tokens from several hierarchy levels (the set is
// described in k_attn_fwd.hip).
#pragma once
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
constexpr int CMP_E = 2048;        // the complement's entries per query block, at most

// Per-wave LDS: two value tiles (160-byte rows), two key tiles (144-byte
// rows) and the table of pooled-entry rows (ECAP ints).  With ECAP = 64 a
// workgroup of 4 waves needs under 40 KB, so 4 workgroups share a CU.
template <int ECAP, int D>
struct FwdLds {
    static constexpr int V_TILE = BS * TileShape<D>::ROW_T;  // bf16 elements
    static constexpr int K_TILE = BS * TileShape<D>::ROW_A;
    static constexpr int PER_WAVE = 2 * V_TILE + 2 * K_TILE + 2 * ECAP;  // in bf16 units
};

// The forward of one query block (qblk over G * n1) by one wave; sm: the
// wave's LDS (FwdLds<ECAP, D>::PER_WAVE elements, 16-byte aligned).
template <int ECAP, int D>
__device__ __forceinline__ void fwd_block(const unsigned short* __restrict__ q,
                                          const unsigned short* __restrict__ k,
                                          const unsigned short* __restrict__ v,
                                          unsigned short* __restrict__ out,
                                          float* __restrict__ lse, const Geo& g, const Ws& w,
                                          long qblk, unsigned short* sm)
{
    using Lay = FwdLds<ECAP, D>;
    using TS = TileShape<D>;
    constexpr int NI = TS::NI;
    const int lane = threadIdx.x & 63;
    const int gq = lane >> 4, nq = lane & 15;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const float c = g.scale * LOG2E;  // logits in log2 units
    const long hbase = (long)gh * g.N * D;
    const long qbase = hbase + (long)i * BS * D;
    bf16x8 bq[NI];  // B operand of S^T: query row lane%16, channels 32u + 8(lane/16) ..
#pragma unroll
    for (int u = 0; u < NI; ++u) bq[u] = ld_bf16x8(q + qbase + nq * D + 32 * u + 8 * gq);
    // the query block's K fine blocks, one per lane (K <= 64).  Causal: the
    // KF valid picks come first, the last of them the block itself (the
    // diagonal tile, masked to keys u <= t), then -1.
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i) * g.K;
    const int rawj = lane < g.K ? sel[lane] : -1;
    const int myj = lane < g.K ? clampi(rawj, g.n[1]) : 0;
    const int KF = g.causal ? max(1, (int)__popcll(__ballot(rawj >= 0))) : g.K;
    // the pooled entries of the enriching levels: rows in the bf16 pooled
    // arrays, with their level (fill_entries)
    int* ent = (int*)(sm + 2 * Lay::V_TILE + 2 * Lay::K_TILE);
    const int E = fill_entries(g, w, gh, i, ent, lane);
    lds_fence();

    Online<D> st;
#pragma unroll
    for (int d = 0; d < D / 16; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.den = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    unsigned short* la = sm;  // value tiles (transposed reads)
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
    const int NF = (g.causal ? KF - 1 : g.K) / 2;  // full (unmasked) fine pairs
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
    // masked tail: tiles t < NFT are the fine tiles left (the lone one of an
    // odd count, and when causal the diagonal one, last), then the pooled
    // tiles; pairs of tiles, rows read through per-lane pointers
    const int NFT = KF - 2 * NF;
    const int NT = NFT + (E + BS - 1) / BS;
    auto tail_off = [&](int t, int r) -> long {
        // element offset of row r (0..15) of tail tile t in k / v (a fine
        // tile) or in the pooled copies; rows past the last entry repeat a
        // valid one (they are masked)
        if (t < NFT) return hbase + ((long)__builtin_amdgcn_readlane(myj, 2 * NF + t) * BS + r) * D;
        return (long)(ent[min(BS * (t - NFT) + r, E - 1)] & ENT_ROW) * D;
    };
    // valid rows of fine tail tile t: all 16, or for the causal diagonal
    // tile those at or before this lane's query row (a per-lane count)
    auto fine_rows = [&](int t) { return (g.causal && t == NFT - 1) ? nq + 1 : BS; };
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
        const int na = t < NFT ? fine_rows(t) : max(0, min(BS, E - BS * (t - NFT)));
        const int nb = t + 1 >= NT ? 0
                     : (t + 1 < NFT ? fine_rows(t + 1) : max(0, min(BS, E - BS * (t + 1 - NFT))));
        float ba[4], bb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ea = BS * (t - NFT) + 4 * gq + r, eb = ea + BS;
            ba[r] = (t < NFT || g.lb2 == 0.f) ? 0.f
                    : g.lb2 * (float)ent_level(ent[max(0, min(ea, E - 1))]);
            bb[r] = (t + 1 < NFT || g.lb2 == 0.f) ? 0.f
                    : g.lb2 * (float)ent_level(ent[max(0, min(eb, E - 1))]);
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

}  // namespace
}  // namespace llsa
