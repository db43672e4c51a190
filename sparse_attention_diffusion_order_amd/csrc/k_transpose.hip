// k_transpose.hip -- sparse index transpose (key block -> query blocks).
//
// LLSA skill summary, "Core Technique" 3: the backward pass needs, for each
// key block, the query blocks that selected it; the pages obtain these lists
// directly from the sparse index lists instead of from a dense mask.
//
// A counting sort into CSR form (rowptr [G][n_l+1], col [G][n_l*K], every
// list ascending), one launch per level, coarsest first.  Below the coarsest
// level the counts come from the selection pass (per block and per 16
// blocks) and each workgroup sums the prefix before its own bins from the
// group counts; at the coarsest level, where every query block is a
// candidate, each workgroup counts the (short) index lists itself.  The fill
// gathers instead of scattering: one workgroup owns 16 sibling key blocks
// 16p .. 16p+15 and walks the only query blocks that can have chosen them --
// at a finer level, the children of the query blocks in the parent level's
// list of block p (hierarchical selection only offers children of chosen
// parents); at the coarsest level, all query blocks.  The candidates are
// walked in ascending order and ballots give each hit its rank, so lists come
// out sorted and identical run to run; the fill uses no atomics.
#include "transpose.h"

namespace llsa {
namespace {

__global__ __launch_bounds__(256) void transpose_fill(Geo g, Ws w, int l, int pair)
{
    transpose_block(g, w, l, pair, blockIdx.x);
}

}  // namespace

TrFirst transpose_first(const Geo& g)
{
    TrFirst f;
    if (g.L >= 2 && g.n[g.L] <= TOP2_MAX) {  // the two coarsest levels in one launch
        f.l = g.L - 1;
        f.pair = 1;
        f.wgs = g.G * ((g.n[g.L] + 15) / 16 + (g.n[g.L - 1] + 15) / 16);
    } else {
        f.l = g.L;
        f.pair = 0;
        f.wgs = g.G * ((g.n[g.L] + 15) / 16);
    }
    return f;
}

hipError_t launch_transpose_after(const Geo& g, const Ws& w, const TrFirst& f, hipStream_t st)
{
    // finer levels need the coarser lists: one launch each, coarsest first
    for (int l = f.l - 1; l >= 1; --l) {
        dim3 grid((unsigned)(g.G * ((g.n[l] + 15) / 16)));
        hipLaunchKernelGGL(transpose_fill, grid, dim3(256), 0, st, g, w, l, 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_transpose(const Geo& g, const Ws& w, hipStream_t st)
{
    // level 1 feeds the key-major dk/dv pass; levels >= 2 feed the pooled-
    // token gradients; finer levels need the coarser lists, so all are built,
    // coarsest first.
    const TrFirst f = transpose_first(g);
    hipLaunchKernelGGL(transpose_fill, dim3((unsigned)f.wgs), dim3(256), 0, st, g, w, f.l, f.pair);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_transpose_after(g, w, f, st);
}

}  // namespace llsa
