// k_transpose.hip -- sparse index transpose (key block -> query blocks).
//
// LLSA skill summary, "Core Technique" 3: the backward pass needs, for each
// key block, the query blocks that selected it; the pages obtain these lists
// directly from the sparse index lists instead of from a dense mask.
//
// Levels are transposed coarsest first, each by count -> prefix scan -> fill
// into CSR form (rowptr [G][n_l+1], col [G][n_l*K], every list ascending).
// The count and fill kernels gather instead of scatter: one workgroup owns 16
// sibling key blocks 16p .. 16p+15 and walks the only query blocks that can
// have chosen them -- at a finer level, the children of the query blocks in
// the parent level's list of block p (hierarchical selection only offers
// children of chosen parents); at the coarsest level, all query blocks.  The
// candidates are walked in ascending order and ballots give each hit its rank,
// so lists come out sorted and identical run to run, with no atomics.
#include "common.h"

namespace llsa {
namespace {

// Candidate query block number c of the wave's group (ascending in c).
struct Cands {
    const int* plist;  // parent level's list of block p (nullptr at the coarsest level)
    int n;             // number of candidates
    __device__ __forceinline__ int row(int c) const
    {
        return plist ? BS * plist[c >> 4] + (c & 15) : c;
    }
};

__device__ __forceinline__ Cands make_cands(const Geo& g, const Ws& w, int l, int gh, int grp)
{
    Cands cs;
    if (l == g.L) {
        cs.plist = nullptr;
        cs.n = g.n[l];
    } else {
        const int* rp = w.rowptr[l] + (long)gh * (g.n[l + 1] + 1);
        cs.plist = w.col[l] + (long)gh * g.n[l + 1] * g.K + rp[grp];
        cs.n = BS * (rp[grp + 1] - rp[grp]);
    }
    return cs;
}

// 16-bit mask of which of the bins 16*grp .. 16*grp+15 query block i selected,
// and in *first the number of its entries below bin 16*grp.  The list is
// ascending, so the hits form one run starting at *first: the hit in bin b
// sits at position *first + popcount(mask & ((1 << b) - 1)).
__device__ __forceinline__ unsigned hit_mask(const int* I, int K, int grp, int* first)
{
    unsigned m = 0;
    int below = 0;
    const int lo = BS * grp;
    if ((K & 3) == 0) {
        for (int e = 0; e < K; e += 4) {
            const int4 j4 = *(const int4*)(I + e);
            m |= ((j4.x >> 4) == grp) ? 1u << (j4.x & 15) : 0u;
            m |= ((j4.y >> 4) == grp) ? 1u << (j4.y & 15) : 0u;
            m |= ((j4.z >> 4) == grp) ? 1u << (j4.z & 15) : 0u;
            m |= ((j4.w >> 4) == grp) ? 1u << (j4.w & 15) : 0u;
            below += (j4.x < lo) + (j4.y < lo) + (j4.z < lo) + (j4.w < lo);
        }
    } else {
        for (int e = 0; e < K; ++e) {
            const int j = I[e];
            m |= ((j >> 4) == grp) ? 1u << (j & 15) : 0u;
            below += j < lo;
        }
    }
    *first = below;
    return m;
}

// One workgroup (4 waves) per 16 sibling key blocks; one candidate query
// block per thread.  FILL == false: rowptr[j + 1] = |T_l[j]|.  FILL == true:
// col lists (and, for the pooled-token gradients, the position of j in each
// listed query block's index list).  Ranks: ballot within a wave, counts of
// lower waves through LDS, counts of earlier rounds carried in registers.
template <bool FILL>
__global__ __launch_bounds__(256) void transpose_pass(Geo g, Ws w, int l)
{
    __shared__ int wcnt[4][16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int groups = (g.n[l] + 15) / 16;
    const int gh = blockIdx.x / groups, grp = blockIdx.x % groups;
    const int* I = w.idx[l - 1] + (long)gh * g.n[l] * g.K;
    int* rowptr = w.rowptr[l - 1] + (long)gh * (g.n[l] + 1);
    int* col = w.col[l - 1] + (long)gh * g.n[l] * g.K;
    unsigned char* slots = w.slot[l - 1] + (long)gh * g.n[l] * g.K;
    const Cands cs = make_cands(g, w, l, gh, grp);
    const unsigned long long below = (1ull << lane) - 1ull;
    int run[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) run[b] = FILL ? rowptr[min(16 * grp + b, g.n[l])] : 0;
    for (int c0 = 0; c0 < cs.n; c0 += 256) {
        const int c = c0 + tid;
        int i = 0, first = 0;
        unsigned m = 0;
        if (c < cs.n) {
            i = cs.row(c);
            m = hit_mask(I + (long)i * g.K, g.K, grp, &first);
        }
        unsigned long long bal[16];
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            bal[b] = __ballot((m >> b) & 1u);
            if (lane == b) wcnt[wv][b] = __popcll(bal[b]);
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            int before = 0, total = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int cnt = wcnt[u][b];
                before += (u < wv) ? cnt : 0;
                total += cnt;
            }
            if (FILL && ((m >> b) & 1u)) {
                const int pos = run[b] + before + __popcll(bal[b] & below);
                col[pos] = i;
                slots[pos] = (unsigned char)(first + __popc(m & ((1u << b) - 1u)));
            }
            run[b] += total;
        }
        __syncthreads();
    }
    if (!FILL && tid < 16 && 16 * grp + tid < g.n[l]) {
        int cnt = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) cnt = (b == tid) ? run[b] : cnt;
        rowptr[16 * grp + tid + 1] = cnt;
    }
}

// rowptr[1..n] holds counts; turn it into the exclusive prefix (rowptr[0] = 0).
__global__ __launch_bounds__(1024) void transpose_scan(Geo g, Ws w, int l)
{
    __shared__ int wsum[16];
    const int n = g.n[l];
    int* rowptr = w.rowptr[l - 1] + (long)blockIdx.x * (n + 1);
    const int per = (n + 1023) / 1024;
    const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
    int s = 0;
    for (int j = lo; j < hi; ++j) s += rowptr[j + 1];
    // inclusive scan of s over the block
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int off = 0;
    for (int k = 0; k < wv; ++k) off += wsum[k];
    int run = off + x - s;  // exclusive prefix of this thread's first bin
    for (int j = lo; j < hi; ++j) {
        int cnt = rowptr[j + 1];
        run += cnt;
        rowptr[j + 1] = run;
    }
    if (threadIdx.x == 0) rowptr[0] = 0;
}

}  // namespace

hipError_t launch_transpose(const Geo& g, const Ws& w, hipStream_t st)
{
    // level 1 feeds the key-major dk/dv pass; levels >= 2 feed the enrichment
    // gradients; finer levels need the coarser lists, so all are built.
    for (int l = g.L; l >= 1; --l) {
        dim3 grid((unsigned)(g.G * ((g.n[l] + 15) / 16)));
        hipLaunchKernelGGL(transpose_pass<false>, grid, dim3(256), 0, st, g, w, l);
        hipLaunchKernelGGL(transpose_scan, dim3(g.G), dim3(1024), 0, st, g, w, l);
        hipLaunchKernelGGL(transpose_pass<true>, grid, dim3(256), 0, st, g, w, l);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace llsa
