// k_zorder.hip -- Z-order (quadtree) token permutation gather, and the grid
// order that extends it to rectangles and video.
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

__device__ __forceinline__ unsigned spread3(unsigned x)  // bit b -> bit 3b (10 bits)
{
    x &= 0x000003ffu;
    x = (x | (x << 16)) & 0xff0000ffu;
    x = (x | (x << 8)) & 0x0300f00fu;
    x = (x | (x << 4)) & 0x030c30c3u;
    x = (x | (x << 2)) & 0x09249249u;
    return x;
}

// CPR_LOG2 >= 0: chunks per row is 2^CPR_LOG2 and every index splits with
// shifts; CPR_LOG2 < 0: any chunk count (divisions).
template <typename V, int CPR_LOG2>
__global__ __launch_bounds__(256) void zorder_kernel(const V* __restrict__ src,
                                                     V* __restrict__ dst, long long total,
                                                     int chunks_per_row, int side_log2,
                                                     int inverse)
{
    const unsigned side_mask = (1u << side_log2) - 1u;
    const unsigned n_mask = (1u << (2 * side_log2)) - 1u;
    for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += (long long)gridDim.x * blockDim.x) {
        long long row;
        int c;
        if (CPR_LOG2 >= 0) {
            row = id >> CPR_LOG2;
            c = (int)(id & ((1 << CPR_LOG2) - 1));
        } else {
            row = id / chunks_per_row;
            c = (int)(id - row * chunks_per_row);
        }
        const long long o = row >> (2 * side_log2);
        const unsigned p = (unsigned)row & n_mask;  // destination position
        unsigned s;                                   // source position
        if (!inverse) {  // p is a Morton code; read the raster cell it names
            unsigned x = gather_bits(p), y = gather_bits(p >> 1);
            s = (y << side_log2) | x;
        } else {  // p is a raster cell; read its Morton position
            unsigned y = p >> side_log2, x = p & side_mask;
            s = (spread_bits(y) << 1) | spread_bits(x);
        }
        const long long srow = (o << (2 * side_log2)) | s;
        dst[id] = src[CPR_LOG2 >= 0 ? (srow << CPR_LOG2) | c : srow * chunks_per_row + c];
    }
}

template <typename V>
__global__ __launch_bounds__(256) void grid_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                   long long total, int cpr, unsigned n,
                                                   GridGeo gg, int inverse)
{
    const int tb = (gg.video ? 3 : 2) * gg.s_log2;  // bits of a position inside a tile
    const unsigned smask = (1u << gg.s_log2) - 1u;
    for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
         id += (long long)gridDim.x * blockDim.x) {
        const long long row = id / cpr;
        const int c = (int)(id - row * cpr);
        const long long o = row / n;
        const unsigned p = (unsigned)(row - o * n);  // destination cell
        unsigned s;                                  // source cell
        if (!inverse) {  // p is a grid-order position: find its raster cell
            s = grid_source(p, gg);
        } else {  // p is a raster cell: find its grid-order position
            const unsigned x = p % gg.W, r = p / gg.W;
            const unsigned y = r % gg.H, t = r / gg.H;
            const unsigned tz = gg.video ? t >> gg.s_log2 : 0u;
            const unsigned tile = (tz * gg.th + (y >> gg.s_log2)) * gg.tw + (x >> gg.s_log2);
            const unsigned code = gg.video ? (spread3(t & smask) << 2) | (spread3(y & smask) << 1) |
                                                 spread3(x & smask)
                                           : (spread_bits(y & smask) << 1) | spread_bits(x & smask);
            s = (tile << tb) | code;
        }
        dst[id] = src[((long long)o * n + s) * cpr + c];
    }
}

}  // namespace

hipError_t launch_grid_order(const void* src, void* dst, long long outer, int frames, int height,
                             int width, int inner_bytes, int inverse, hipStream_t st)
{
    if (frames == 1 && height == width && (width & (width - 1)) == 0)  // one square tile
        return launch_zorder(src, dst, outer, width, inner_bytes, inverse, st);
    const GridGeo gg = make_grid_geo(frames, height, width);
    const int vw = (inner_bytes % 16 == 0) ? 16 : (inner_bytes % 8 == 0) ? 8 : 4;
    const int cpr = inner_bytes / vw;
    const unsigned n = (unsigned)frames * (unsigned)height * (unsigned)width;
    const long long total = outer * (long long)n * cpr;
    long long blocks = (total + 255) / 256;
    if (blocks > (1ll << 20)) blocks = 1ll << 20;
    dim3 grid((unsigned)blocks);
    if (vw == 16)
        hipLaunchKernelGGL(grid_kernel<uint4>, grid, dim3(256), 0, st, (const uint4*)src,
                           (uint4*)dst, total, cpr, n, gg, inverse);
    else if (vw == 8)
        hipLaunchKernelGGL(grid_kernel<uint2>, grid, dim3(256), 0, st, (const uint2*)src,
                           (uint2*)dst, total, cpr, n, gg, inverse);
    else
        hipLaunchKernelGGL(grid_kernel<unsigned>, grid, dim3(256), 0, st, (const unsigned*)src,
                           (unsigned*)dst, total, cpr, n, gg, inverse);
    return hipGetLastError();
}

hipError_t launch_zorder(const void* src, void* dst, long long outer, int side, int inner_bytes,
                         int inverse, hipStream_t st)
{
    int lg = 0;
    while ((1 << lg) < side) ++lg;
    int vw = (inner_bytes % 16 == 0) ? 16 : (inner_bytes % 8 == 0) ? 8 : 4;
    int cpr = inner_bytes / vw;
    long long total = outer * ((long long)side * side) * cpr;
    long long blocks = (total + 255) / 256;
    if (blocks > (1ll << 20)) blocks = 1ll << 20;
    dim3 grid((unsigned)blocks);
    const int pl = (cpr & (cpr - 1)) == 0 ? __builtin_ctz(cpr) : -1;
#define LLSA_ZLAUNCH(V, L)                                                                  \
    hipLaunchKernelGGL((zorder_kernel<V, L>), grid, dim3(256), 0, st, (const V*)src, (V*)dst, \
                       total, cpr, lg, inverse)
    if (vw == 16) {
        if (pl == 3) LLSA_ZLAUNCH(uint4, 3);
        else if (pl == 2) LLSA_ZLAUNCH(uint4, 2);
        else if (pl == 4) LLSA_ZLAUNCH(uint4, 4);
        else LLSA_ZLAUNCH(uint4, -1);
    } else if (vw == 8) {
        LLSA_ZLAUNCH(uint2, -1);
    } else {
        LLSA_ZLAUNCH(unsigned, -1);
    }
#undef LLSA_ZLAUNCH
    return hipGetLastError();
}

}  // namespace llsa
