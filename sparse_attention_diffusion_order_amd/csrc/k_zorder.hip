// k_zorder.hip -- Z-order (quadtree) token permutation gather.
//
// LLSA README, "reordering non-sequential data": tokens of a 2-D grid are
// reordered so that at every scale the quadrants come top-left, top-right,
// bottom-left, bottom-right, i.e. the Morton code with the row bit above the
// column bit.  The kernel computes the code by bit interleaving; no table.
// Each thread moves one VW-byte chunk; consecutive threads write consecutive
// destination bytes, and every source row is read whole by adjacent threads.
#include "common.h"

namespace llsa {
namespace {

__device__ __forceinline__ unsigned spread_bits(unsigned x)  // 0bABCD -> 0b0A0B0C0D
{
    x &= 0x0000ffffu;
    x = (x | (x << 8)) & 0x00ff00ffu;
    x = (x | (x << 4)) & 0x0f0f0f0fu;
    x = (x | (x << 2)) & 0x33333333u;
    x = (x | (x << 1)) & 0x55555555u;
    return x;
}

__device__ __forceinline__ unsigned gather_bits(unsigned x)  // inverse of spread_bits
{
    x &= 0x55555555u;
    x = (x | (x >> 1)) & 0x33333333u;
    x = (x | (x >> 2)) & 0x0f0f0f0fu;
    x = (x | (x >> 4)) & 0x00ff00ffu;
    x = (x | (x >> 8)) & 0x0000ffffu;
    return x;
}

template <typename V>
__global__ __launch_bounds__(256) void zorder_kernel(const V* __restrict__ src,
                                                     V* __restrict__ dst, long long total,
                                                     int chunks_per_row, int side_log2,
                                                     long long n, int inverse)
{
    const unsigned side_mask = (1u << side_log2) - 1u;
    for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += (long long)gridDim.x * blockDim.x) {
        long long row = id / chunks_per_row;
        int c = (int)(id - row * chunks_per_row);
        long long o = row / n;
        unsigned p = (unsigned)(row - o * n);  // destination position
        unsigned s;                             // source position
        if (!inverse) {  // p is a Morton code; read the raster cell it names
            unsigned x = gather_bits(p), y = gather_bits(p >> 1);
            s = (y << side_log2) | x;
        } else {  // p is a raster cell; read its Morton position
            unsigned y = p >> side_log2, x = p & side_mask;
            s = (spread_bits(y) << 1) | spread_bits(x);
        }
        dst[id] = src[(o * n + s) * chunks_per_row + c];
    }
}

}  // namespace

hipError_t launch_zorder(const void* src, void* dst, long long outer, int side, int inner_bytes,
                         int inverse, hipStream_t st)
{
    int lg = 0;
    while ((1 << lg) < side) ++lg;
    long long n = (long long)side * side;
    int vw = (inner_bytes % 16 == 0) ? 16 : (inner_bytes % 8 == 0) ? 8 : 4;
    int cpr = inner_bytes / vw;
    long long total = outer * n * cpr;
    long long blocks = (total + 255) / 256;
    if (blocks > (1ll << 20)) blocks = 1ll << 20;
    dim3 grid((unsigned)blocks);
    if (vw == 16)
        hipLaunchKernelGGL(zorder_kernel<uint4>, grid, dim3(256), 0, st, (const uint4*)src,
                           (uint4*)dst, total, cpr, lg, n, inverse);
    else if (vw == 8)
        hipLaunchKernelGGL(zorder_kernel<uint2>, grid, dim3(256), 0, st, (const uint2*)src,
                           (uint2*)dst, total, cpr, lg, n, inverse);
    else
        hipLaunchKernelGGL(zorder_kernel<unsigned>, grid, dim3(256), 0, st,
                           (const unsigned*)src, (unsigned*)dst, total, cpr, lg, n, inverse);
    return hipGetLastError();
}

}  // namespace llsa
