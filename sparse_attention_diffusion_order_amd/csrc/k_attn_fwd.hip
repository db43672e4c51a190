// k_attn_fwd.hip -- sparse attention forward with hierarchical KV enrichment.
//
// LLSA README, usage: a drop-in for non-causal scaled-dot-product attention;
// skill summary, "Core Technique" 2: the key/value set of a query is enriched
// with coarse (pooled) tokens from several hierarchy levels.
//
// Key/value set of the 16 tokens of query block i (level-l ancestor
// a_l = i / 16^(l-1)):
//   - the 16*K tokens of the key blocks idx_1[i] (fine tiles, 16 keys each);
//   - for every level l = 1..L the pooled pairs (kbar_l[j], vbar_l[j]) for
//     j in idx_l[a_l] (unless LLSA_NO_ENRICH).
// One softmax over the whole set, scale 1/sqrt(d); lse in natural log.
//
// The pooled entries of all levels (L*K of them) form extra tiles of 16,
// read from the bf16 copy of the pyramid that the pool pass writes.
//
// bf16 kernel (MFMA): one wave per query block, 4 waves per workgroup.
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, A = key rows, B = query rows;
//                    lane (g = lane/16, n = lane%16) holds S^T[4g + r][n]:
//                    four keys of query n, so softmax statistics of query n
//                    are reduced over lanes n, n+16, n+32, n+48 only.
//   O^T += V^T P^T   A = V^T from LDS with ds_read_b64_tr_b16 (values are
//                    staged row-major, read back transposed), B = P^T taken
//                    straight from the S^T accumulator layout: two 16-key
//                    tiles form the 32-deep contraction.
// fp32 kernel (VALU): one thread per query token, explicit pooled tokens.
#include "common.h"

namespace llsa {
namespace {

// Staged 16-row tiles in LDS.  Rows read back transposed (ds_read_b64_tr_b16,
// 4 rows x 32 B per 16 lanes) use a 160-byte stride; rows read as MFMA
// operands (ds_read_b128, 8 rows x 16 B per 8 lanes) a 144-byte stride: both
// spread their accesses over all 32 banks.
constexpr int LDS_ROW = 80;   // transposed-read tiles
constexpr int ROW_A = 72;     // operand-read tiles
constexpr int TILE_ELEMS = BS * LDS_ROW;

__device__ __forceinline__ bf16x8 ld_bf16x8(const unsigned short* p)
{
    return *(const bf16x8*)p;
}

// Registers of one prefetched pair of fine tiles: rows vr and vr+8 (columns
// vc .. vc+7) of the key and value tiles a and b.  Every load instruction
// covers 8 whole 128-byte rows, the fast gather pattern of the vector L1.
struct FinePair {
    bf16x8 ka0, ka1, kb0, kb1;
    bf16x8 va0, va1, vb0, vb1;
};

template <int ROW>
__device__ __forceinline__ void stage_rows(unsigned short* lds, bf16x8 r0, bf16x8 r1, int lane)
{
    const int vr = lane >> 3, vc = (lane & 7) * 8;
    *(bf16x8*)(lds + vr * ROW + vc) = r0;
    *(bf16x8*)(lds + (vr + 8) * ROW + vc) = r1;
}

// A operand of S^T = K Q^T from a staged key tile: row lane%16, channels
// 8(lane/16) .. +7 and 32 + 8(lane/16) .. +7.
__device__ __forceinline__ void key_operand(const unsigned short* lds, bf16x8& k0, bf16x8& k1,
                                            int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
    k0 = *(const bf16x8*)(lds + nq * ROW_A + 8 * gq);
    k1 = *(const bf16x8*)(lds + nq * ROW_A + 32 + 8 * gq);
}

// Softmax state.  The exponentials use a reference max m that is raised only
// when a new logit exceeds it by more than TAU (log2 units), so P <= 2^TAU and
// the accumulators are rarely rescaled; the result is the same softmax.
constexpr float TAU = 8.0f;

struct Online {
    f32x4 acc[4];  // O^T tiles: lane holds O^T[16d + 4(lane/16) + r][query lane%16]
    float m;       // reference max (log2 units), equal in the 4 lanes of a query
    float lsum;    // this lane's share of the softmax denominator
};

// One step over two 16-entry tiles whose values are staged in LDS at la / lb.
// na / nb: valid entries (MASK == false: both tiles full).
template <bool MASK>
__device__ __forceinline__ void attend_pair(Online& st, bf16x8 bq0, bf16x8 bq1, bf16x8 ka0,
                                            bf16x8 ka1, bf16x8 kb0, bf16x8 kb1,
                                            const unsigned short* la, const unsigned short* lb,
                                            int na, int nb, float c, int lane)
{
    const int gq = lane >> 4;
    const int rr = (lane & 15) >> 2, xx = lane & 3;
    const f32x4 zero = {};
    const f32x4 sa = mfma32(ka1, bq1, mfma32(ka0, bq0, zero));
    const f32x4 sb = mfma32(kb1, bq1, mfma32(kb0, bq0, zero));
    float ya[4], yb[4];  // raw scores, masked entries at -inf
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        ya[r] = (!MASK || 4 * gq + r < na) ? sa[r] : -INFINITY;
        yb[r] = (!MASK || 4 * gq + r < nb) ? sb[r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(ya[0], ya[1]), fmaxf(ya[2], ya[3])),
                     fmaxf(fmaxf(yb[0], yb[1]), fmaxf(yb[2], yb[3])));
    mx = max_x4(mx) * c;
    if (__ballot(mx > st.m + TAU)) {
        const float mnew = fmaxf(st.m, mx);
        const float alpha = fast_exp2(st.m - mnew);
        st.lsum *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) st.acc[d] *= alpha;
        st.m = mnew;
    }
    const float nm = -st.m;
    bf16x8 pp;
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float pa = fast_exp2(fmaf(ya[r], c, nm));
        const float pb = fast_exp2(fmaf(yb[r], c, nm));
        ls += pa + pb;
        pp[r] = (bf16)pa;
        pp[4 + r] = (bf16)pb;
    }
    st.lsum += ls;
    lds_fence();
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
        bf16x4 va = lds_read_tr(la + off), vb = lds_read_tr(lb + off);
        bf16x8 av = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
        st.acc[d] = mfma32(av, pp, st.acc[d]);
    }
}

constexpr int MAX_E = MAX_L * 64;  // pooled entries per query block (L * K)

// Per-wave LDS: two value tiles (160-byte rows), two key tiles (144-byte
// rows) and the table of pooled-entry rows (ECAP ints).  With ECAP = 64 a
// workgroup of 4 waves needs under 40 KB, so 4 workgroups share a CU.
template <int ECAP>
struct FwdLds {
    static constexpr int V_TILE = BS * LDS_ROW;  // bf16 elements
    static constexpr int K_TILE = BS * ROW_A;
    static constexpr int PER_WAVE = 2 * V_TILE + 2 * K_TILE + 2 * ECAP;  // in bf16 units
};

template <int ECAP>
__global__ __launch_bounds__(256) void attn_fwd_bf16(const unsigned short* __restrict__ q,
                                                     const unsigned short* __restrict__ k,
                                                     const unsigned short* __restrict__ v,
                                                     unsigned short* __restrict__ out,
                                                     float* __restrict__ lse, Geo g, Ws w)
{
    using Lay = FwdLds<ECAP>;
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][Lay::PER_WAVE];
    const int lane = threadIdx.x & 63, wv = uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)xcd_block(blockIdx.x, gridDim.x) * 4 + wv;  // over G * n1
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const float c = g.scale * LOG2E;  // logits in log2 units
    const long hbase = (long)gh * g.N * D;
    const long qbase = hbase + (long)i * BS * D;
    const bf16x8 bq0 = ld_bf16x8(q + qbase + nq * D + 8 * gq);
    const bf16x8 bq1 = ld_bf16x8(q + qbase + nq * D + 32 + 8 * gq);
    // the query block's K fine blocks, one per lane (K <= 64)
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + i) * g.K;
    const int myj = lane < g.K ? sel[lane] : 0;
    // pooled entries e = (l-1)*K + slot: their rows in the bf16 pooled arrays
    const int E = (g.flags & LLSA_NO_ENRICH) ? 0 : g.L * g.K;
    int* ent = (int*)(smem[wv] + 2 * Lay::V_TILE + 2 * Lay::K_TILE);
    for (int l = 1; l <= (E ? g.L : 0); ++l) {
        const long a = (long)gh * g.n[l] + (i >> (4 * (l - 1)));
        for (int s0 = 0; s0 < g.K; s0 += 64)
            if (s0 + lane < g.K)
                ent[(l - 1) * g.K + s0 + lane] =
                    (int)(w.prow[l - 1] + (long)gh * g.n[l] + w.idx[l - 1][a * g.K + s0 + lane]);
    }
    lds_fence();

    Online st;
#pragma unroll
    for (int d = 0; d < 4; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.lsum = 0.f;
    unsigned short* la = smem[wv];  // value tiles (transposed reads)
    unsigned short* lb = la + Lay::V_TILE;
    unsigned short* lka = lb + Lay::V_TILE;  // key tiles (operand reads)
    unsigned short* lkb = lka + Lay::K_TILE;

    // One pipeline over all tile pairs: NF pairs of fine tiles, then NP - NF
    // pairs of pooled tiles.  The next pair's loads are in flight while this
    // one is computed (two register sets alternate).  Loads are issued
    // unconditionally -- out-of-range tiles re-read a valid row and are
    // masked -- so the compiler's wait counts stay exact.
    const int NF = (g.K + 1) / 2;
    const int NT = (E + BS - 1) / BS;  // pooled tiles
    const int NP = NF + (NT + 1) / 2;
    const int vr = lane >> 3, vc = (lane & 7) * 8;
    auto load_pair = [&](FinePair& f, int p) {
        long ka, kb, ka8, kb8;  // element offsets of rows vr and vr + 8
        const unsigned short *kp, *vp;
        if (p < NF) {
            const int ja = __builtin_amdgcn_readlane(myj, min(2 * p, g.K - 1));
            const int jb = __builtin_amdgcn_readlane(myj, min(2 * p + 1, g.K - 1));
            ka = hbase + ((long)ja * BS + vr) * D + vc;
            kb = hbase + ((long)jb * BS + vr) * D + vc;
            ka8 = ka + 8 * D;
            kb8 = kb + 8 * D;
            kp = k;
            vp = v;
        } else {
            const int t = 2 * (p - NF);
            ka = (long)ent[min(BS * t + vr, E - 1)] * D + vc;
            ka8 = (long)ent[min(BS * t + vr + 8, E - 1)] * D + vc;
            kb = (long)ent[min(BS * t + BS + vr, E - 1)] * D + vc;
            kb8 = (long)ent[min(BS * t + BS + vr + 8, E - 1)] * D + vc;
            kp = w.kb16;
            vp = w.vb16;
        }
        f.ka0 = ld_bf16x8(kp + ka);
        f.ka1 = ld_bf16x8(kp + ka8);
        f.va0 = ld_bf16x8(vp + ka);
        f.va1 = ld_bf16x8(vp + ka8);
        f.kb0 = ld_bf16x8(kp + kb);
        f.kb1 = ld_bf16x8(kp + kb8);
        f.vb0 = ld_bf16x8(vp + kb);
        f.vb1 = ld_bf16x8(vp + kb8);
    };
    auto step = [&](const FinePair& f, int p) {
        stage_rows<ROW_A>(lka, f.ka0, f.ka1, lane);
        stage_rows<ROW_A>(lkb, f.kb0, f.kb1, lane);
        stage_rows<LDS_ROW>(la, f.va0, f.va1, lane);
        stage_rows<LDS_ROW>(lb, f.vb0, f.vb1, lane);
        lds_fence();
        bf16x8 ka0, ka1, kb0, kb1;
        key_operand(lka, ka0, ka1, lane);
        key_operand(lkb, kb0, kb1, lane);
        if (p < NF && g.K > 1) {
            attend_pair<false>(st, bq0, bq1, ka0, ka1, kb0, kb1, la, lb, BS, BS, c, lane);
        } else {
            const int e0 = p < NF ? 0 : BS * 2 * (p - NF);
            const int na = p < NF ? BS : max(0, min(BS, E - e0));
            const int nb = p < NF ? 0 : max(0, min(BS, E - e0 - BS));
            attend_pair<true>(st, bq0, bq1, ka0, ka1, kb0, kb1, la, lb, na, nb, c, lane);
        }
    };
    FinePair A, B;
    load_pair(A, 0);
    for (int p = 0;; p += 2) {
        load_pair(B, min(p + 1, NP - 1));
        step(A, p);
        if (p + 1 >= NP) break;
        load_pair(A, min(p + 2, NP - 1));
        step(B, p + 1);
        if (p + 2 >= NP) break;
    }

    const float lsum = sum_x4(st.lsum);
    const float inv = 1.0f / lsum;
    const long obase = qbase + nq * D + 4 * gq;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        u16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = f2bf(st.acc[d][r] * inv);
        *(u16x4*)(out + obase + 16 * d) = o;
    }
    if (gq == 0) lse[(long)gh * g.N + (long)i * BS + nq] = (st.m + fast_log2(lsum)) * LN2;
}

// ------------------------------------------------------------ fp32 path

__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    float* __restrict__ out,
                                                    float* __restrict__ lse, Geo g, Ws w)
{
    const long tg = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (tg >= (long)g.G * g.N) return;
    const int gh = (int)(tg / g.N), t = (int)(tg % g.N);
    float qr[D], o[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = q[tg * D + c];
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    auto visit = [&](const float* kr, const float* vr) {
        float z = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) z = fmaf(qr[c], kr[c], z);
        z *= g.scale;
        if (z > m) {
            float a = expf(m - z);
            l *= a;
#pragma unroll
            for (int c = 0; c < D; ++c) o[c] *= a;
            m = z;
        }
        float p = expf(z - m);
        l += p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = fmaf(p, vr[c], o[c]);
    };
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + t / BS) * g.K;
    for (int s = 0; s < g.K; ++s)
        for (int r = 0; r < BS; ++r) {
            long row = ((long)gh * g.N + (long)sel[s] * BS + r) * D;
            visit(k + row, v + row);
        }
    if (!(g.flags & LLSA_NO_ENRICH))
        for (int lv = 1; lv <= g.L; ++lv) {
            const int a = t >> (4 * lv);
            const int* sl = w.idx[lv - 1] + ((long)gh * g.n[lv] + a) * g.K;
            for (int s = 0; s < g.K; ++s) {
                long row = ((long)gh * g.n[lv] + sl[s]) * D;
                visit(w.kbar[lv - 1] + row, w.vbar[lv - 1] + row);
            }
        }
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) out[tg * D + c] = o[c] * inv;
    lse[tg] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                           int dtype, const Geo& g, const Ws& w, hipStream_t st)
{
    if (dtype == LLSA_BF16) {
        long nblk = (long)g.G * g.n[1];
        auto kern = (g.L * g.K <= 64) ? attn_fwd_bf16<64> : attn_fwd_bf16<MAX_E>;
        hipLaunchKernelGGL(kern, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, (unsigned short*)out, lse, g, w);
    } else {
        long ntok = (long)g.G * g.N;
        hipLaunchKernelGGL(attn_fwd_f32, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, (float*)out, lse,
                           g, w);
    }
    return hipGetLastError();
}

}  // namespace llsa
