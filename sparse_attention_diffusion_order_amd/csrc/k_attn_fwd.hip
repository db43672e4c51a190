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
// for its 16^l keys.  LLSA_CAUSAL (a reading; the README's usage names the
// non-causal form only): idx_1[i] holds block i itself (last of its valid
// picks), masked to keys u <= t, and the pooled token of an ancestor's own
// block is left out; unused slots (-1) are skipped.
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
#include "attn_block.h"

namespace llsa {
namespace {

template <int ECAP, int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16(const unsigned short* __restrict__ q,
                                                     const unsigned short* __restrict__ k,
                                                     const unsigned short* __restrict__ v,
                                                     unsigned short* __restrict__ out,
                                                     float* __restrict__ lse, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][FwdLds<ECAP, D>::PER_WAVE];
    const int wv = uniform(threadIdx.x >> 6);
    const long qblk = (long)xcd_block(blockIdx.x, gridDim.x, g.xcd_chunk) * 4 + wv;  // over G * n1
    if (qblk >= (long)g.G * g.n[1]) return;
    fwd_block<ECAP, D>(q, k, v, out, lse, g, w, qblk, smem[wv]);
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
    const long qb0 = ((long)xcd_block(blockIdx.x, gridDim.x, g.xcd_chunk) * 4 + wv) * 4;  // over G * n1
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

// one wave per query token; keys in batches of 16 (for_each_batch, lane =
// key r + 16 channel group), the online softmax updated once per batch
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse, Geo g, Ws w)
{
    constexpr int CH = D / 4;
    const long tg = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (tg >= (long)g.G * g.N) return;
    const int lane = threadIdx.x & 63, r = lane & 15;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    float qc[CH], o[CH];
    load_slice<D>(qc, q + tg * D, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) o[c] = 0.f;
    float m = -INFINITY, l = 0.f;  // l, o: this lane's rows' share
    auto run = [&](const RowBatch& bt) {
        float kx[CH], vx[CH];
        load_slice<D>(kx, bt.k, lane);
        load_slice<D>(vx, bt.v, lane);
        const float z = r < bt.n ? slice_dot<D>(qc, kx) * g.scale + bt.bias : -INFINITY;
        const float mb = row16_max(z);
        if (mb > m) {
            const float a = expf(m - mb);
            l *= a;
#pragma unroll
            for (int c = 0; c < CH; ++c) o[c] *= a;
            m = mb;
        }
        const float p = expf(z - m);
        l += p;
#pragma unroll
        for (int c = 0; c < CH; ++c) o[c] = fmaf(p, vx[c], o[c]);
    };
    for_each_batch<D>(g, w, k, v, gh, t, lane, run);
    l = row16_sum(l);
#pragma unroll
    for (int c = 0; c < CH; ++c) o[c] = row16_sum(o[c]);
    if (r == 0) {
        float4* dst = (float4*)(out + tg * D + CH * (lane >> 4));
#pragma unroll
        for (int u = 0; u < CH / 4; ++u)
            dst[u] = float4{o[4 * u] / l, o[4 * u + 1] / l, o[4 * u + 2] / l, o[4 * u + 3] / l};
    }
    if (lane == 0) lse[tg] = m + logf(l);
}

template <int D>
hipError_t launch_attn_fwd_d(const void* q, const void* k, const void* v, void* out, float* lse,
                             int dtype, const Geo& g, const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        // the four-block kernel (d = 64): every fine list and every pooled
        // list fit one 16-entry tile, and the launch fills the chip at least
        // twice over at its 2 waves per SIMD (2048 waves a round); with fewer
        // query blocks the one-block kernel's 4 waves per SIMD win (measured:
        // 64^2 x 12 heads 15.6 against 28.0 us, 128^2 x 12 heads 51.7
        // against 60.9 us; 256^2 x 6 heads 105 against 97 us)
        bool fits = D == D64 && g.K <= BS && g.n[1] % 4 == 0 && !g.cmp && !g.causal &&
                    nblk / 4 >= 2 * 2048;
        for (int l = g.l0; l <= g.L; ++l) fits = fits && g.Kl[l] <= BS;
        if (fits) {
            hipLaunchKernelGGL(attn_fwd_u4, dim3((unsigned)((nblk + 15) / 16)), dim3(256), 0, st,
                               (const unsigned short*)q, (const unsigned short*)k,
                               (const unsigned short*)v, (unsigned short*)out, lse, g, w);
        } else {
            const int me = g.max_pooled();
            auto kern = me <= 64 ? attn_fwd_bf16<64, D>
                      : me <= MAX_E ? attn_fwd_bf16<MAX_E, D> : attn_fwd_bf16<CMP_E, D>;
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
