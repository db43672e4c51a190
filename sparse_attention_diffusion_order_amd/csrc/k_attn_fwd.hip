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
// read from the float32 pyramid and rounded to bf16 for the MFMA.
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

__device__ __forceinline__ bf16x8 ld_f32_as_bf16x8(const float* p)
{
    float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    bf16x8 r;
    r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
    r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
    return r;
}

// Pooled entry e (0 .. L*K-1) of query block i: level 1 + e / K, slot e % K
// of the index list of the query's ancestor at that level.
__device__ __forceinline__ long enrich_row(const Geo& g, const Ws& w, int gh, int i, int e,
                                           int* level)
{
    int l = 1 + e / g.K, s = e % g.K;
    int a = i >> (4 * (l - 1));
    int j = w.idx[l - 1][((long)gh * g.n[l] + a) * g.K + s];
    *level = l;
    return ((long)gh * g.n[l] + j) * D;
}

// Pooled-entry tile t (entries 16t .. 16t+15): A operand of S^T (rows =
// entries) into k0/k1, value rows into LDS (row-major, zero rows for masked
// entries).  Returns the number of valid entries.
__device__ __forceinline__ int fetch_enrich(const Geo& g, const Ws& w, int gh, int i, int t,
                                            unsigned short* lds, bf16x8& k0, bf16x8& k1,
                                            int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
    const int vr = lane >> 3, vc = (lane & 7) * 8;
    const int e0 = t * BS;
    const int nvalid = max(0, min(BS, g.L * g.K - e0));
    const bf16x8 z = {};
    k0 = z;
    k1 = z;
    if (nq < nvalid) {
        int lv;
        long off = enrich_row(g, w, gh, i, e0 + nq, &lv);
        k0 = ld_f32_as_bf16x8(w.kbar[lv - 1] + off + 8 * gq);
        k1 = ld_f32_as_bf16x8(w.kbar[lv - 1] + off + 32 + 8 * gq);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int row = vr + 8 * h;
        bf16x8 val = z;
        if (row < nvalid) {
            int lv;
            long off = enrich_row(g, w, gh, i, e0 + row, &lv);
            val = ld_f32_as_bf16x8(w.vbar[lv - 1] + off + vc);
        }
        *(bf16x8*)(lds + row * LDS_ROW + vc) = val;
    }
    return nvalid;
}


// Registers of one prefetched pair of fine tiles: rows vr and vr+8 (columns
// vc .. vc+7) of the key and value tiles a and b.  Every load instruction
// covers 8 whole 128-byte rows, the fast gather pattern of the vector L1.
struct FinePair {
    bf16x8 ka0, ka1, kb0, kb1;
    bf16x8 va0, va1, vb0, vb1;
};

__device__ __forceinline__ void load_fine(FinePair& f, const unsigned short* k,
                                          const unsigned short* v, long hbase, int ja, int jb,
                                          int lane)
{
    const int vr = lane >> 3, vc = (lane & 7) * 8;
    const long a = hbase + (long)ja * BS * D + vr * D + vc;
    const long b = hbase + (long)max(jb, 0) * BS * D + vr * D + vc;
    f.ka0 = ld_bf16x8(k + a);
    f.ka1 = ld_bf16x8(k + a + 8 * D);
    f.va0 = ld_bf16x8(v + a);
    f.va1 = ld_bf16x8(v + a + 8 * D);
    f.kb0 = ld_bf16x8(k + b);
    f.kb1 = ld_bf16x8(k + b + 8 * D);
    f.vb0 = ld_bf16x8(v + b);
    f.vb1 = ld_bf16x8(v + b + 8 * D);
}

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

__global__ __launch_bounds__(256) void attn_fwd_bf16(const unsigned short* __restrict__ q,
                                                     const unsigned short* __restrict__ k,
                                                     const unsigned short* __restrict__ v,
                                                     unsigned short* __restrict__ out,
                                                     float* __restrict__ lse, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][4][TILE_ELEMS];
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
    const int myj = lane < g.K ? sel[lane] : -1;

    Online st;
#pragma unroll
    for (int d = 0; d < 4; ++d) st.acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.lsum = 0.f;
    unsigned short* la = smem[wv][0];  // value tiles (transposed reads)
    unsigned short* lb = smem[wv][1];
    unsigned short* lka = smem[wv][2];  // key tiles (operand reads)
    unsigned short* lkb = smem[wv][3];

    // fine tiles, two per step; the next pair's loads are in flight meanwhile.
    // Two register sets alternate; prefetches are unconditional (indices
    // clamped to the last block) so the compiler's wait counts stay exact.
    auto jsel = [&](int t) { return __builtin_amdgcn_readlane(myj, min(t, g.K - 1)); };
    auto step = [&](const FinePair& f, bool full) {
        stage_rows<ROW_A>(lka, f.ka0, f.ka1, lane);
        stage_rows<ROW_A>(lkb, f.kb0, f.kb1, lane);
        stage_rows<LDS_ROW>(la, f.va0, f.va1, lane);
        stage_rows<LDS_ROW>(lb, f.vb0, f.vb1, lane);
        lds_fence();
        bf16x8 ka0, ka1, kb0, kb1;
        key_operand(lka, ka0, ka1, lane);
        key_operand(lkb, kb0, kb1, lane);
        if (full)
            attend_pair<false>(st, bq0, bq1, ka0, ka1, kb0, kb1, la, lb, BS, BS, c, lane);
        else
            attend_pair<true>(st, bq0, bq1, ka0, ka1, kb0, kb1, la, lb, BS, 0, c, lane);
    };
    if (g.K == 1) {
        FinePair A;
        load_fine(A, k, v, hbase, jsel(0), jsel(0), lane);
        step(A, false);
    } else {
        const int npairs = g.K / 2;
        FinePair A, B;
        load_fine(A, k, v, hbase, jsel(0), jsel(1), lane);
        for (int p = 0;; p += 2) {
            load_fine(B, k, v, hbase, jsel(2 * p + 2), jsel(2 * p + 3), lane);
            step(A, true);
            if (p + 1 >= npairs) break;
            load_fine(A, k, v, hbase, jsel(2 * p + 4), jsel(2 * p + 5), lane);
            step(B, true);
            if (p + 2 >= npairs) break;
        }
    }
    // pooled tokens of every level
    if (!(g.flags & LLSA_NO_ENRICH)) {
        const int nt = (g.L * g.K + BS - 1) / BS;
        for (int t = 0; t < nt; t += 2) {
            bf16x8 ka0, ka1, kb0, kb1;
            int na = fetch_enrich(g, w, gh, i, t, la, ka0, ka1, lane);
            int nb = fetch_enrich(g, w, gh, i, t + 1, lb, kb0, kb1, lane);
            attend_pair<true>(st, bq0, bq1, ka0, ka1, kb0, kb1, la, lb, na, nb, c, lane);
        }
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
        hipLaunchKernelGGL(attn_fwd_bf16, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st,
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
