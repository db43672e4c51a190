// k_pool.hip -- block mean-pool pyramid of Q, K and V.
//
// LLSA skill summary, "Core Technique" 1 (hierarchical compression) and the
// arXiv abstract (block-wise representation of tokens): the level-l token i
// is the mean of the tokens block i covers -- its 16 level-(l-1) children
// 16i .. 16i+15, fewer for the partial last block of a level when 16^l does
// not divide N (the children then weighted by the tokens each covers).
// Levels are computed recursively, in float32.
//
// With GATHER the pass also performs the grid-order gather (LLSA README,
// reordering of non-sequential data): q, k, v are read in raster order, each
// token from the raster cell its grid-order position names, and the
// grid-ordered copies are written as the pass goes -- the same bytes as
// llsa_grid_order, and the same sums, without reading the tensors twice.
//
// pool_l12: one workgroup per 256 consecutive tokens of one head and one
// tensor.  Thread (blk, sub) sums the 16 tokens of level-1 block blk over the
// d/16 channels (d/16) sub .. (d/16)(sub+1) - 1, so a token row is read whole
// by 16 adjacent lanes with one load each (8 or 16 bytes in bf16).  Level 2
// (one block per workgroup) is the mean of the 16 level-1 means, formed in
// LDS.  pool_up forms levels >= 3 from level l-1.
// The pooled keys and values are also stored rounded to bf16 (the operands
// the attention kernels feed to the MFMA).  pool_l12 also zeroes the
// selection's pick counters when given them (llsa_forward), which saves the
// selection pass a launch.
#include "common.h"

namespace llsa {
namespace {

// C consecutive channels (C = 4 or 8) of one token row: load() reads them
// raw (one 8- or 16-byte load in bf16, one or two 16-byte loads in fp32),
// add() widens them to float and adds them to s.  load_once() is load() with
// the nontemporal hint, for the raster rows of the gathering pass: they are
// read once, and streaming them keeps the caches for the grid-ordered copies
// the selection and attention read next (256x256: forward with the gather
// 0.185 -> 0.182 ms).
template <typename T, int C> struct Row;
template <int C> struct Row<float, C> {
    float4 r[C / 4];
    __device__ __forceinline__ void load(const float* p)
    {
#pragma unroll
        for (int h = 0; h < C / 4; ++h) r[h] = ((const float4*)p)[h];
    }
    __device__ __forceinline__ void add(float (&s)[C]) const
    {
#pragma unroll
        for (int h = 0; h < C / 4; ++h) {
            s[4 * h] += r[h].x; s[4 * h + 1] += r[h].y; s[4 * h + 2] += r[h].z; s[4 * h + 3] += r[h].w;
        }
    }
    __device__ __forceinline__ void load_once(const float* p)
    {
#pragma unroll
        for (int h = 0; h < C / 4; ++h) {
            const f32x4 x = __builtin_nontemporal_load((const f32x4*)p + h);
            r[h] = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
    __device__ __forceinline__ void store(float* p) const
    {
#pragma unroll
        for (int h = 0; h < C / 4; ++h) ((float4*)p)[h] = r[h];
    }
};
template <int C> struct Row<unsigned short, C> {
    unsigned u[C / 2];  // two bf16 per word, the lower channel in the low half
    __device__ __forceinline__ void load(const unsigned short* p)
    {
        if constexpr (C == 4) {
            const uint2 x = *(const uint2*)p;
            u[0] = x.x; u[1] = x.y;
        } else {
            const uint4 x = *(const uint4*)p;
            u[0] = x.x; u[1] = x.y; u[2] = x.z; u[3] = x.w;
        }
    }
    __device__ __forceinline__ void load_once(const unsigned short* p)
    {
        typedef unsigned uv __attribute__((ext_vector_type(C / 2)));
        const uv x = __builtin_nontemporal_load((const uv*)p);
#pragma unroll
        for (int h = 0; h < C / 2; ++h) u[h] = x[h];
    }
    __device__ __forceinline__ void add(float (&s)[C]) const
    {
#pragma unroll
        for (int h = 0; h < C / 2; ++h) {
            s[2 * h] += __uint_as_float(u[h] << 16);
            s[2 * h + 1] += __uint_as_float(u[h] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ void store(unsigned short* p) const
    {
        if constexpr (C == 4)
            *(uint2*)p = make_uint2(u[0], u[1]);
        else
            *(uint4*)p = make_uint4(u[0], u[1], u[2], u[3]);
    }
};

// Raster sources and grid-ordered destinations of the gathering pass.
template <typename T>
struct Gather {
    T* q;
    T* k;
    T* v;
    GridGeo gg;
};

template <typename T, int D, bool GATHER>
__global__ __launch_bounds__(256) void pool_l12(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, Geo g, Ws w,
                                                Gather<T> gt)
{
    constexpr int C = D / 16;  // channels per thread: C sub .. C sub + C - 1
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
    float s[C];
#pragma unroll
    for (int c = 0; c < C; ++c) s[c] = 0.f;
    if (live) {
        const T* p = x + ((long)gh * g.N + (long)(b0 + blk) * BS) * D + C * sub;
        Row<T, C> r[BS];
        if (GATHER) {
            // token (b0 + blk) 16 + t of the head comes from the raster cell
            // its grid position names; its grid-ordered copy goes to position.
            // When a tile holds at least 16 cells, the block's 16 positions
            // differ in the low four bits of the in-tile code only: x0 y0 x1
            // y1 (image) or x0 y0 t0 x1 (video), offsets from the first cell.
            const T* src = x + (long)gh * g.N * D + C * sub;
            const unsigned p0 = (unsigned)(b0 + blk) * BS;
            const GridGeo& gg = gt.gg;
            if ((gg.video ? 3 : 2) * gg.s_log2 >= 4) {
                const long base = grid_source(p0, gg);
#pragma unroll
                for (int t = 0; t < BS; ++t) {
                    const unsigned b0_ = t & 1, b1_ = (t >> 1) & 1, b2_ = (t >> 2) & 1,
                                   b3_ = (t >> 3) & 1;
                    const long off = gg.video
                                         ? ((long)b2_ * gg.H + b1_) * gg.W + (b0_ | (b3_ << 1))
                                         : (long)(b1_ | (b3_ << 1)) * gg.W + (b0_ | (b2_ << 1));
                    r[t].load_once(src + (base + off) * D);
                }
            } else {
#pragma unroll
                for (int t = 0; t < BS; ++t) r[t].load_once(src + (long)grid_source(p0 + t, gg) * D);
            }
            T* dst = (tensor == 0 ? gt.q : tensor == 1 ? gt.k : gt.v) +
                     ((long)gh * g.N + (long)(b0 + blk) * BS) * D + C * sub;
#pragma unroll
            for (int t = 0; t < BS; ++t) r[t].store(dst + (long)t * D);
        } else {
#pragma unroll
            for (int t = 0; t < BS; ++t) r[t].load(p + (long)t * D);
        }
#pragma unroll
        for (int t = 0; t < BS; ++t) r[t].add(s);
        const float inv = 1.0f / BS;
        const long row = (long)gh * n1 + b0 + blk;
#pragma unroll
        for (int c = 0; c < C; ++c) s[c] *= inv;
#pragma unroll
        for (int h = 0; h < C / 4; ++h)
            *(float4*)(lv1 + row * D + C * sub + 4 * h) =
                make_float4(s[4 * h], s[4 * h + 1], s[4 * h + 2], s[4 * h + 3]);
        if (tensor) {
            unsigned short* dst = (tensor == 1 ? w.kb16 : w.vb16) + (w.prow[0] + row) * D + C * sub;
#pragma unroll
            for (int h = 0; h < C / 4; ++h) {
                const u16x4 o = {f2bf(s[4 * h]), f2bf(s[4 * h + 1]), f2bf(s[4 * h + 2]),
                                 f2bf(s[4 * h + 3])};
                *(u16x4*)(dst + 4 * h) = o;
            }
        }
    }
    if (g.L >= 2) {  // b0 is a multiple of 16, so this workgroup is one level-2 block
#pragma unroll
        for (int c = 0; c < C; ++c) m1[blk][C * sub + c] = s[c];
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

// gq, gk, gv != nullptr: q, k, v are raster-order sources, gathered into gq,
// gk, gv in grid order (GridGeo gg) by the same pass
template <int D>
hipError_t launch_pool_d(const void* q, const void* k, const void* v, void* gq, void* gk,
                         void* gv, const GridGeo& gg, int dtype, const Geo& g, const Ws& w,
                         hipStream_t st)
{
    dim3 grid(g.G * ((g.n[1] + 15) / 16), 3);
    if (dtype == LLSA_BF16) {
        using T = unsigned short;
        const Gather<T> gt{(T*)gq, (T*)gk, (T*)gv, gg};
        auto kern = gq ? pool_l12<T, D, true> : pool_l12<T, D, false>;
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const T*)q, (const T*)k, (const T*)v,
                           g, w, gt);
    } else {
        using T = float;
        const Gather<T> gt{(T*)gq, (T*)gk, (T*)gv, gg};
        auto kern = gq ? pool_l12<T, D, true> : pool_l12<T, D, false>;
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const T*)q, (const T*)k, (const T*)v,
                           g, w, gt);
    }
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
    const GridGeo gg{};
    return g.d == D128 ? launch_pool_d<D128>(q, k, v, nullptr, nullptr, nullptr, gg, dtype, g, wz, st)
                       : launch_pool_d<D64>(q, k, v, nullptr, nullptr, nullptr, gg, dtype, g, wz, st);
}

hipError_t launch_pool_gather(const void* qr, const void* kr, const void* vr, void* q, void* k,
                              void* v, const GridGeo& gg, int dtype, const Geo& g, const Ws& w,
                              hipStream_t st)
{
    return g.d == D128 ? launch_pool_d<D128>(qr, kr, vr, q, k, v, gg, dtype, g, w, st)
                       : launch_pool_d<D64>(qr, kr, vr, q, k, v, gg, dtype, g, w, st);
}

}  // namespace llsa
