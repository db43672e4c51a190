// k_pool.hip -- block mean-pool pyramid of Q, K and V.
//
// LLSA skill summary, "Core Technique" 1 (hierarchical compression) and the
// arXiv abstract (block-wise representation of tokens): the level-l token i
// is the mean of the tokens block i covers -- its 16 level-(l-1) children
// 16i .. 16i+15, fewer for the partial last block of a level when 16^l does
// not divide N (the children then weighted by the tokens each covers).
// Levels are computed recursively, in float32.
//
// pool_l12: one workgroup per 256 consecutive tokens of one head and one
// tensor.  Thread (blk, sub) sums the 16 tokens of level-1 block blk over the
// channels 4*sub .. 4*sub+3 (and 64 + 4*sub .. when d = 128), so each 64-channel
// part of a token row is read whole by 16 adjacent lanes.  Level 2 (one block per workgroup) is the mean of the
// 16 level-1 means, formed in LDS.  pool_up forms levels >= 3 from level l-1.
// The pooled keys and values are also stored rounded to bf16 (the operands
// the attention kernels feed to the MFMA).  pool_l12 also zeroes the
// selection's pick counters when given them (llsa_forward), which saves the
// selection pass a launch.
#include "common.h"

namespace llsa {
namespace {

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ float4 load(const float* p)
    {
        return *(const float4*)p;
    }
};
template <> struct Vec4<unsigned short> {
    static __device__ __forceinline__ float4 load(const unsigned short* p)
    {
        uint2 u = *(const uint2*)p;
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
};

__device__ __forceinline__ void put_bf16x4(unsigned short* dst, long off, float4 s)
{
    u16x4 o = {f2bf(s.x), f2bf(s.y), f2bf(s.z), f2bf(s.w)};
    *(u16x4*)(dst + off) = o;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_l12(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, Geo g, Ws w)
{
    constexpr int NC = D / 64;  // 4-channel groups per thread: channels 4 sub + 64 c
    __shared__ float m1[16][D];
    if (w.cnt_all) {
        // zero the selection's pick counters (the selection pass that follows
        // adds to them); far fewer counters than threads
        const long nth = (long)gridDim.x * gridDim.y * blockDim.x;
        for (long t = ((long)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
             t < w.cnt_len; t += nth)
            w.cnt_all[t] = 0;
    }
    const int tensor = blockIdx.y;
    const T* x = tensor == 0 ? q : tensor == 1 ? k : v;
    float* lv1 = tensor == 0 ? w.qbar[0] : tensor == 1 ? w.kbar[0] : w.vbar[0];
    float* lv2 = g.L >= 2 ? (tensor == 0 ? w.qbar[1] : tensor == 1 ? w.kbar[1] : w.vbar[1])
                          : nullptr;
    const int n1 = g.n[1];
    const int wg_per_head = (n1 + 15) / 16;
    const int gh = blockIdx.x / wg_per_head;
    const int b0 = (blockIdx.x % wg_per_head) * 16;  // first level-1 block
    const int blk = threadIdx.x >> 4, sub = threadIdx.x & 15;
    const bool live = b0 + blk < n1;
    float4 s[NC];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) s[cg] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        const T* p = x + ((long)gh * g.N + (long)(b0 + blk) * BS) * D + 4 * sub;
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
            float4 r[BS];
#pragma unroll
            for (int t = 0; t < BS; ++t) r[t] = Vec4<T>::load(p + (long)t * D + 64 * cg);
#pragma unroll
            for (int t = 0; t < BS; ++t) {
                s[cg].x += r[t].x;
                s[cg].y += r[t].y;
                s[cg].z += r[t].z;
                s[cg].w += r[t].w;
            }
        }
        const float inv = 1.0f / BS;
        const long row = (long)gh * n1 + b0 + blk;
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
            s[cg] = make_float4(s[cg].x * inv, s[cg].y * inv, s[cg].z * inv, s[cg].w * inv);
            *(float4*)(lv1 + row * D + 4 * sub + 64 * cg) = s[cg];
            if (tensor)
                put_bf16x4(tensor == 1 ? w.kb16 : w.vb16, (w.prow[0] + row) * D + 4 * sub + 64 * cg,
                           s[cg]);
        }
    }
    if (g.L >= 2) {  // b0 is a multiple of 16, so this workgroup is one level-2 block
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
            m1[blk][4 * sub + 64 * cg + 0] = s[cg].x;
            m1[blk][4 * sub + 64 * cg + 1] = s[cg].y;
            m1[blk][4 * sub + 64 * cg + 2] = s[cg].z;
            m1[blk][4 * sub + 64 * cg + 3] = s[cg].w;
        }
        __syncthreads();
        if (threadIdx.x < D) {
            // the mean of the tokens of the level-2 block: its level-1 blocks
            // (whole blocks of 16 tokens; a partial last level-2 block has
            // fewer of them, and the others hold zeros)
            float a = 0.f;
#pragma unroll
            for (int b = 0; b < 16; ++b) a += m1[b][threadIdx.x];
            const int live1 = min(16, n1 - b0);
            const float mean = a / (float)live1;
            const long row = (long)gh * g.n[2] + b0 / 16;
            lv2[row * D + threadIdx.x] = mean;
            if (tensor)
                (tensor == 1 ? w.kb16 : w.vb16)[(w.prow[1] + row) * D + threadIdx.x] = f2bf(mean);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void pool_up(Geo g, Ws w, int l)
{
    const int tensor = blockIdx.y;
    const float* src = (tensor == 0 ? w.qbar : tensor == 1 ? w.kbar : w.vbar)[l - 2];
    float* dst = (tensor == 0 ? w.qbar : tensor == 1 ? w.kbar : w.vbar)[l - 1];
    long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
    long total = (long)g.G * g.n[l] * D;
    if (id >= total) return;
    long row = id / D;
    int c = (int)(id % D);
    // the mean of the tokens the block covers: its existing children, each
    // weighted by the tokens it covers (all 16^(l-1) unless it is the partial
    // last one; equal power-of-two weights give the plain mean exactly)
    const int gh = (int)(row / g.n[l]), i = (int)(row % g.n[l]);
    const int np = g.n[l - 1];
    float a = 0.f, wsum = 0.f;
    for (int t = 0; t < BS && BS * i + t < np; ++t) {
        const float wt = (float)g.tokens(l - 1, BS * i + t);
        a += wt * src[((long)gh * np + BS * i + t) * D + c];
        wsum += wt;
    }
    const float mean = a / wsum;
    dst[id] = mean;
    if (tensor) (tensor == 1 ? w.kb16 : w.vb16)[(w.prow[l - 1] + row) * D + c] = f2bf(mean);
}

template <int D>
hipError_t launch_pool_d(const void* q, const void* k, const void* v, int dtype, const Geo& g,
                         const Ws& w, hipStream_t st)
{
    dim3 grid(g.G * ((g.n[1] + 15) / 16), 3);
    if (dtype == LLSA_BF16)
        hipLaunchKernelGGL((pool_l12<unsigned short, D>), grid, dim3(256), 0, st,
                           (const unsigned short*)q, (const unsigned short*)k,
                           (const unsigned short*)v, g, w);
    else
        hipLaunchKernelGGL((pool_l12<float, D>), grid, dim3(256), 0, st, (const float*)q,
                           (const float*)k, (const float*)v, g, w);
    hipError_t e = hipGetLastError();
    for (int l = 3; l <= g.L && e == hipSuccess; ++l) {
        long total = (long)g.G * g.n[l] * D;
        hipLaunchKernelGGL(pool_up<D>, dim3((unsigned)((total + 255) / 256), 3), dim3(256), 0, st,
                           g, w, l);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, const void* v, int dtype, const Geo& g,
                       const Ws& w, bool zero_counts, hipStream_t st)
{
    Ws wz = w;
    if (!zero_counts) wz.cnt_all = nullptr;
    return g.d == D128 ? launch_pool_d<D128>(q, k, v, dtype, g, wz, st)
                       : launch_pool_d<D64>(q, k, v, dtype, g, wz, st);
}

}  // namespace llsa
