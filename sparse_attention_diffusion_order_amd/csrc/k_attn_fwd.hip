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
// Level-1 pooled tokens are folded into the fine tiles: kbar_1[j] is the mean
// of the 16 keys of block j, so its logit is the mean of that tile's 16
// logits and its value contributes P_e/16 to each of the tile's 16 values.
// No extra loads or MFMAs are needed for them.  Levels >= 2 form extra tiles
// of 16 pooled entries.
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

constexpr int LDS_ROW = 80;  // bf16 per staged row: 64 + 16 pad (160 B, spreads banks)
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

// Enrichment entry e (0 .. (L-1)*K-1) of query block i: level 2 + e / K,
// slot e % K of the index list of the query's ancestor at that level.
__device__ __forceinline__ long enrich_row(const Geo& g, const Ws& w, int gh, int i, int e,
                                           int* level)
{
    int l = 2 + e / g.K, s = e % g.K;
    int a = i >> (4 * (l - 1));
    int j = w.idx[l - 1][((long)gh * g.n[l] + a) * g.K + s];
    *level = l;
    return ((long)gh * g.n[l] + j) * D;
}

// Fetch one 16-entry tile: the A operand of S^T (rows = entries) into k0/k1
// and the value rows into LDS (row-major, zero rows for masked entries).
// Returns the number of valid entries (16 for fine tiles).
__device__ __forceinline__ int fetch_tile(const Geo& g, const Ws& w, const unsigned short* k,
                                          const unsigned short* v, int gh, int i, int t,
                                          int ntiles, unsigned short* lds, bf16x8& k0,
                                          bf16x8& k1, int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
    const int vr = lane >> 3, vc = (lane & 7) * 8;  // staging: rows vr, vr+8; cols vc..vc+7
    if (t < g.K) {  // fine tile: key block idx_1[i][t]
        int j = w.idx[0][((long)gh * g.n[1] + i) * g.K + t];
        long base = ((long)gh * g.N + (long)j * BS) * D;
        k0 = ld_bf16x8(k + base + nq * D + 8 * gq);
        k1 = ld_bf16x8(k + base + nq * D + 32 + 8 * gq);
        bf16x8 v0 = ld_bf16x8(v + base + vr * D + vc);
        bf16x8 v1 = ld_bf16x8(v + base + (vr + 8) * D + vc);
        *(bf16x8*)(lds + vr * LDS_ROW + vc) = v0;
        *(bf16x8*)(lds + (vr + 8) * LDS_ROW + vc) = v1;
        return BS;
    }
    const int E = (t < ntiles && !(g.flags & LLSA_NO_ENRICH)) ? (g.L - 1) * g.K : 0;
    const int e0 = (t - g.K) * BS;
    const int nvalid = max(0, min(BS, E - e0));
    bf16x8 z = {};
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

__global__ __launch_bounds__(256) void attn_fwd_bf16(const unsigned short* __restrict__ q,
                                                     const unsigned short* __restrict__ k,
                                                     const unsigned short* __restrict__ v,
                                                     unsigned short* __restrict__ out,
                                                     float* __restrict__ lse, Geo g, Ws w)
{
    __shared__ __attribute__((aligned(16))) unsigned short smem[4][2][TILE_ELEMS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gq = lane >> 4, nq = lane & 15;
    const long qblk = (long)blockIdx.x * 4 + wv;  // over G * n1
    if (qblk >= (long)g.G * g.n[1]) return;
    const int gh = (int)(qblk / g.n[1]), i = (int)(qblk % g.n[1]);
    const bool enrich = !(g.flags & LLSA_NO_ENRICH);
    const float c = g.scale * LOG2E;  // logits in log2 units

    const long qbase = ((long)gh * g.N + (long)i * BS) * D;
    const bf16x8 bq0 = ld_bf16x8(q + qbase + nq * D + 8 * gq);
    const bf16x8 bq1 = ld_bf16x8(q + qbase + nq * D + 32 + 8 * gq);

    const int ntiles = g.K + (enrich ? ((g.L - 1) * g.K + BS - 1) / BS : 0);
    f32x4 acc[4] = {};
    float m = -INFINITY, lsum = 0.f;
    unsigned short* la = smem[wv][0];
    unsigned short* lb = smem[wv][1];
    const int rr = (lane & 15) >> 2, xx = lane & 3;  // transposed-read coordinates

    for (int ta = 0; ta < ntiles; ta += 2) {
        const int tb = ta + 1;
        bf16x8 ka0, ka1, kb0, kb1;
        int na = fetch_tile(g, w, k, v, gh, i, ta, ntiles, la, ka0, ka1, lane);
        int nb = fetch_tile(g, w, k, v, gh, i, tb, ntiles, lb, kb0, kb1, lane);
        const f32x4 zero = {};
        f32x4 sa = mfma32(ka1, bq1, mfma32(ka0, bq0, zero));
        f32x4 sb = mfma32(kb1, bq1, mfma32(kb0, bq0, zero));
        float za[4], zb[4], mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            za[r] = (4 * gq + r < na) ? sa[r] * c : -INFINITY;
            zb[r] = (4 * gq + r < nb) ? sb[r] * c : -INFINITY;
            mx = fmaxf(mx, fmaxf(za[r], zb[r]));
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] *= alpha;
        float pa[4], pb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pa[r] = fast_exp2(za[r] - m);
            pb[r] = fast_exp2(zb[r] - m);
        }
        if (enrich) {  // level-1 pooled token of each fine tile, folded in
            if (ta < g.K) {
                float s = za[0] + za[1] + za[2] + za[3];
                s += shfl_xor(s, 16);
                s += shfl_xor(s, 32);
                float pe = fast_exp2(s * (1.0f / BS) - m) * (1.0f / BS);
#pragma unroll
                for (int r = 0; r < 4; ++r) pa[r] += pe;
            }
            if (tb < g.K) {
                float s = zb[0] + zb[1] + zb[2] + zb[3];
                s += shfl_xor(s, 16);
                s += shfl_xor(s, 32);
                float pe = fast_exp2(s * (1.0f / BS) - m) * (1.0f / BS);
#pragma unroll
                for (int r = 0; r < 4; ++r) pb[r] += pe;
            }
        }
        bf16x8 pp;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lsum += pa[r] + pb[r];
            pp[r] = (bf16)pa[r];
            pp[4 + r] = (bf16)pb[r];
        }
        wave_lds_sync();
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int off = (4 * gq + rr) * LDS_ROW + 16 * d + 4 * xx;
            bf16x4 va = lds_read_tr(la + off), vb = lds_read_tr(lb + off);
            bf16x8 av = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
            acc[d] = mfma32(av, pp, acc[d]);
        }
        wave_lds_sync();
    }
    lsum += shfl_xor(lsum, 16);
    lsum += shfl_xor(lsum, 32);
    const float inv = 1.0f / lsum;
    const long obase = qbase + nq * D + 4 * gq;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        u16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = f2bf(acc[d][r] * inv);
        *(u16x4*)(out + obase + 16 * d) = o;
    }
    if (gq == 0) lse[(long)gh * g.N + (long)i * BS + nq] = (m + fast_log2(lsum)) * LN2;
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
