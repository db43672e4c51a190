// transpose.h -- the sparse index transpose of one workgroup (see
// k_transpose.hip), shared by its own launch and by the dQ launch that
// carries the first transpose launch's workgroups.
#pragma once
#include "common.h"

namespace llsa {
namespace {

// Candidate query block number c of the wave's group (ascending in c).
struct Cands {
    const int* plist;  // parent level's list of block p (nullptr at the coarsest level)
    int n;             // number of candidates
    int np;            // blocks of the parent level (bound of a list entry)
    __device__ __forceinline__ int row(int c) const
    {
        return plist ? BS * clampi(plist[c >> 4], np) + (c & 15) : c;
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
        const int tot = g.n[l + 1] * g.Kl[l + 1];
        const int b = clampi(rp[grp], tot + 1), e = max(b, clampi(rp[grp + 1], tot + 1));
        cs.plist = w.col[l] + (long)gh * tot + b;
        cs.n = BS * (e - b);
        cs.np = g.n[l + 1];
    }
    return cs;
}

// 16-bit mask of which of the bins 16*grp .. 16*grp+15 query block i selected,
// and in *first the number of its entries below bin 16*grp.  The list is
// ascending, so the hits form one run starting at *first: the hit in bin b
// sits at position *first + popcount(mask & ((1 << b) - 1)).  Unused slots
// (-1, after the picks of a causal row) are neither hits nor below.
__device__ __forceinline__ unsigned hit_mask(const int* I, int K, int grp, int* first)
{
    unsigned m = 0;
    int below = 0;
    const unsigned lo = BS * grp;
    if ((K & 3) == 0) {
        for (int e = 0; e < K; e += 4) {
            const int4 j4 = *(const int4*)(I + e);
            m |= ((j4.x >> 4) == grp) ? 1u << (j4.x & 15) : 0u;
            m |= ((j4.y >> 4) == grp) ? 1u << (j4.y & 15) : 0u;
            m |= ((j4.z >> 4) == grp) ? 1u << (j4.z & 15) : 0u;
            m |= ((j4.w >> 4) == grp) ? 1u << (j4.w & 15) : 0u;
            below += ((unsigned)j4.x < lo) + ((unsigned)j4.y < lo) + ((unsigned)j4.z < lo) +
                     ((unsigned)j4.w < lo);
        }
    } else {
        for (int e = 0; e < K; ++e) {
            const int j = I[e];
            m |= ((j >> 4) == grp) ? 1u << (j & 15) : 0u;
            below += (unsigned)j < lo;
        }
    }
    *first = below;
    return m;
}

// One workgroup (4 waves) per 16 sibling key blocks 16p .. 16p+15; one
// candidate query block per thread.  Below the coarsest level the selection
// pass counted how often each key block was chosen (per block and per 16
// blocks); the workgroup sums the group counts before its own blocks (n_l / 16
// at most) to get its first CSR position (at the coarsest level it counts
// from the index lists), writes rowptr for its blocks, and fills their
// lists.  Ranks: ballot within a wave, counts of lower waves through LDS,
// counts of earlier rounds in LDS.  Besides col it records, for
// the pooled-token gradients and dk/dv, the position of j in each listed
// query block's index list.
//
// pair != 0: one launch builds the two coarsest levels.  The first
// G * ceil(n_L / 16) workgroups take level L; the others take level L-1 and
// find the level-L blocks that chose their group's parent by scanning the
// level-L index lists (at most TOP2_MAX rows, read from L2) instead of
// reading level L's key->query lists, which the same launch is building.
constexpr int TOP2_MAX = 1024;

__device__ __forceinline__ void transpose_block(const Geo& g, const Ws& w, int l, int pair,
                                                int bid)
{
    __shared__ int wcnt[2][4][16];                   // per round parity, wave, bin
    __shared__ unsigned long long wbal[2][4][16];    // the wave's ballot of each bin
    __shared__ int wsum[4];
    __shared__ int run[16];                          // next free position of each bin
    __shared__ int lcnt[16];
    __shared__ int pickers[TOP2_MAX];                // pair mode: level-L choosers of the parent
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (pair) {
        const int top_wgs = g.G * ((g.n[g.L] + 15) / 16);
        l = bid < top_wgs ? g.L : g.L - 1;
        if (bid >= top_wgs) bid -= top_wgs;
    }
    const int n = g.n[l];
    const int groups = (n + 15) / 16;
    const int gh = bid / groups, grp = bid % groups;
    const int K = g.Kl[l];  // picks per level-l row
    const int* I = w.idx[l - 1] + (long)gh * n * K;
    const int* cnt = w.cnt[l - 1] + (long)gh * n;
    const int* c16 = w.c16[l - 1] + (long)gh * ((n + 15) / 16);
    int* rowptr = w.rowptr[l - 1] + (long)gh * (n + 1);
    int* col = w.col[l - 1] + (long)gh * n * K;
    unsigned char* slots = w.slot[l - 1] + (long)gh * n * K;

    // the candidate walk (parent list -> candidate rows -> their picks) and
    // the prefix over earlier bins are independent: both go out before the
    // first barrier
    Cands cs;
    if (pair && l == g.L - 1) {
        // the level-L rows whose lists hold block grp, ascending
        const int nT = g.n[g.L], KT = g.Kl[g.L];
        const int* IT = w.idx[g.L - 1] + (long)gh * nT * KT;
        const unsigned long long lower = (1ull << lane) - 1ull;
        int total = 0;
        for (int a0 = 0; a0 < nT; a0 += 256) {
            const int a = a0 + tid;
            bool hit = false;
            if (a < nT) {
                const int* row = IT + (long)a * KT;
                if ((KT & 3) == 0) {
                    for (int e = 0; e < KT; e += 4) {
                        const int4 j4 = *(const int4*)(row + e);
                        hit |= (j4.x == grp) | (j4.y == grp) | (j4.z == grp) | (j4.w == grp);
                    }
                } else {
                    for (int e = 0; e < KT; ++e) hit |= row[e] == grp;
                }
            }
            const unsigned long long bal = __ballot(hit);
            if (lane == 0) wsum[wv] = __popcll(bal);
            __syncthreads();
            int pos = total + __popcll(bal & lower);
            for (int u = 0; u < wv; ++u) pos += wsum[u];
            if (hit) pickers[pos] = a;
            total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
            __syncthreads();
        }
        cs.plist = pickers;
        cs.n = BS * total;
        cs.np = g.n[g.L];
    } else {
        cs = make_cands(g, w, l, gh, grp);
    }
    int ci = 0, cfirst = 0;
    unsigned cm = 0;
    auto probe = [&](int c0) {
        const int c = c0 + tid;
        ci = 0;
        cfirst = 0;
        cm = 0;
        if (c < cs.n) {
            ci = cs.row(c);
            // a child past the level's last block (the parent may be the
            // partial last block) does not exist and chose nothing
            if (ci < n) cm = hit_mask(I + (long)ci * K, K, grp, &cfirst);
        }
    };
    probe(0);
    // first position of this group: the counts of blocks 0 .. 16 grp - 1.
    // Below the coarsest level they come from the selection pass, summed as
    // 16-block groups.  At the coarsest level every query block is a
    // candidate, so the workgroup counts them from the (short) index lists:
    // the entries below bin 16 grp, and the hits of each of its 16 bins.
    const bool top = l == g.L;
    int acc = 0;
    if (top) {
        if (tid < 16) lcnt[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += blockDim.x) {
            int below;
            unsigned m = hit_mask(I + (long)i * K, K, grp, &below);
            acc += below;
            for (; m; m &= m - 1) atomicAdd(&lcnt[__ffs(m) - 1], 1);
        }
    } else {
        for (int b = tid; b < grp; b += blockDim.x) acc += c16[b];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) wsum[wv] = acc;
    __syncthreads();
    if (tid < 16) {
        const int base = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        const int j = 16 * grp + tid;
        const int c = top ? lcnt[tid] : j < n ? cnt[j] : 0;
        int x = c;  // inclusive scan over the 16 bins
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(x, o, 16);
            if (tid >= o) x += y;
        }
        run[tid] = base + x - c;
        if (j < n) rowptr[j] = base + x - c;
        if (j == n - 1) rowptr[n] = base + x;
    }
    __syncthreads();

    // Fill, 256 candidates a round.  Every bin's hits are ranked by ballot
    // (candidate order = thread order); a lane then places only its own hits
    // (about one per round): position = the bin's next free slot + the hits
    // of lower waves + the lower lanes of its own wave.  The counts and
    // ballots alternate between two buffers, so the bins' running positions
    // can be advanced after the round while the next round's ballots go in.
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int c0 = 0, par = 0; c0 < cs.n; c0 += 256, par ^= 1) {
        const int i = ci, first = cfirst;
        const unsigned m = cm;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const unsigned long long bal = __ballot((m >> b) & 1u);
            if (lane == b) {
                wcnt[par][wv][b] = __popcll(bal);
                wbal[par][wv][b] = bal;
            }
        }
        probe(c0 + 256);  // the next round's candidates, in flight meanwhile
        __syncthreads();
        for (unsigned mm = m; mm; mm &= mm - 1) {
            const int b = __ffs(mm) - 1;
            int pos = run[b] + __popcll(wbal[par][wv][b] & below);
            for (int u = 0; u < wv; ++u) pos += wcnt[par][u][b];
            // pos < n K whenever the counts match the index lists (both come
            // from the same selection pass); the test only keeps a workspace
            // that was not filled by one from being written out of bounds
            if ((unsigned)pos < (unsigned)(n * K)) {
                col[pos] = i;
                slots[pos] = (unsigned char)(first + __popc(m & ((1u << b) - 1u)));
            }
        }
        __syncthreads();  // every lane has read run[] for this round
        if (tid < 16)
            run[tid] += wcnt[par][0][tid] + wcnt[par][1][tid] + wcnt[par][2][tid] +
                        wcnt[par][3][tid];
    }
}

}  // namespace
}  // namespace llsa
