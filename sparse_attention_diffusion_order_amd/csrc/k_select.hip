// k_select.hip -- hierarchical Top-K block selection.
//
// LLSA skill summary, "Core Technique" 1: Top-K is dense only at the coarsest
// level; every finer level scores only the children of the blocks chosen one
// level up ("progressively adopting sparse Top-K selection with the indices
// found at the previous level"), which makes selection log-linear instead of
// quadratic (arXiv abstract: single-level selection is quadratic).
//
// Score of query block i and key block j: s * <qbar_l[i], kbar_l[j]> in
// float32 (s = 1/sqrt(d)); order: score descending, then block index
// ascending; the K winners are stored in ascending block order.
//
// One workgroup (4 waves) per group of R query rows that share a candidate
// list: the 16 siblings of a parent below the coarsest level (candidates =
// the 16 K' children of the parent's K' picks, ascending), or R rows of the
// coarsest level (candidates = all blocks).  Scores of the R x M tile live in
// LDS.  Each kernel sums a score's channels in one fixed order (stated at the
// kernel), so the result does not depend on the launch.
// Each wave then selects for its rows with an MSB-first radix search on the
// keys (order-preserving integer images of the scores) for a threshold that
// admits exactly the K winners, ballots for ties at the K-th key (lowest
// candidate position first) and a ballot prefix count to write the winners
// in ascending order.  Below the coarsest level the picks are also counted
// per key block and per 16 key blocks (see flush_counts), which the sparse
// transpose uses.  When both fit, the two coarsest levels run in one launch
// (select_top2).
//
// LLSA_CAUSAL (a reading: the README's usage names the non-causal form only):
// a row's own block scores +inf and the candidates after it -inf, so the
// top-K holds the block itself and its best K-1 earlier candidates.  A row
// keeps only candidates with a finite or +inf score: when it has fewer than
// K, the slots after its picks hold -1, and the children of a -1 parent slot
// are no candidates.
#include "common.h"

namespace llsa {
namespace {

// Zero the choice counts of every level (the selection launches that follow
// on the same stream add to them), so each selection pass counts afresh; used
// by the selection part on its own (llsa_forward's pool launch zeroes them).
__global__ __launch_bounds__(256) void clear_counts(int* __restrict__ cnt, long n)
{
    for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < n;
         t += (long)gridDim.x * blockDim.x)
        cnt[t] = 0;
}

__device__ __forceinline__ unsigned order_key(float f)
{
    unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// order_key(-inf): keys at or below it belong to no candidate (no such
// child, or a causal row's later blocks)
constexpr unsigned KEY_NONE = 0x007FFFFFu;

// Block number of candidate c of a row below the coarsest level: child c % 16
// of parent pick pr; an unused parent slot (pr < 0) has no children (INT_MAX,
// past every level's last block)
__device__ __forceinline__ int child_of(int pr, int c, int np)
{
    return pr < 0 ? INT_MAX : BS * clampi(pr, np) + (c % BS);
}

// Causal score of candidate block j in row `row` (row < 0: not causal)
__device__ __forceinline__ float causal_score(float s, int j, int row)
{
    return row < 0 ? s : j == row ? INFINITY : j > row ? -INFINITY : s;
}

// Pick counts of one head below the coarsest level: per key block and per
// 16 key blocks.  A workgroup first counts its picks per candidate in LDS
// (pc), then adds them with one global atomic per picked block and one per
// group of 16 candidates (16 consecutive candidates are always the 16
// children of one block).  Integer atomics: exact whatever the order.
struct Counts {
    int* c1;
    int* c16;
};

__device__ __forceinline__ void flush_counts(const int* pc, const int* cand, int M, Counts cnt)
{
    if (!cnt.c1) return;  // the coarsest level is not counted (its transpose counts itself)
    for (int c = threadIdx.x; c < M; c += blockDim.x)
        if (pc[c]) atomicAdd(cnt.c1 + cand[c], pc[c]);
    for (int gi = threadIdx.x; gi * BS < M; gi += blockDim.x) {
        int sum = 0;
        for (int u = 0; u < BS && gi * BS + u < M; ++u) sum += pc[gi * BS + u];
        if (sum) atomicAdd(cnt.c16 + (cand[gi * BS] >> 4), sum);
    }
}

// Top-K of each of `rows` score rows (LDS, [rows][M]) written ascending to
// out[r * K ..]; one wave per row at a time.  cand: the candidates' block
// numbers (LDS), or nullptr for 0 .. M-1; pc: per-candidate pick counts
// (LDS) to add to, or nullptr; lout: an LDS copy of the output, or nullptr.
template <int KPL>
__device__ __forceinline__ void select_rows(const float* sc, const int* cand, int* out, int rows,
                                            int M, int Kq, int* pc, int* lout = nullptr)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int r = wv; r < rows; r += blockDim.x / 64) {
        unsigned key[KPL];
        bool ok[KPL];
        int nvalid = 0;
#pragma unroll
        for (int s = 0; s < KPL; ++s) {
            int p = s * 64 + lane;
            ok[s] = p < M;
            key[s] = ok[s] ? order_key(sc[r * M + p]) : 0u;
            nvalid += __popcll(__ballot(key[s] > KEY_NONE));
        }
        // the picks this row can make (K, but for a causal row with fewer
        // candidates); -1 in the slots after them
        const int K = min(Kq, nvalid);
        int* orow = out + (long)r * Kq;
        for (int p = K + lane; p < Kq; p += 64) {
            orow[p] = -1;
            if (lout) lout[r * Kq + p] = -1;
        }
        // MSB-first search for a threshold T with #(key >= T) >= K.  It ends
        // at the K-th largest key, or earlier as soon as exactly K keys are
        // >= T: those K keys are then the winners and T splits them from the
        // rest (this is the common case; exact ties run to the last bit).
        unsigned T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            unsigned t = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int s = 0; s < KPL; ++s) cnt += __popcll(__ballot(ok[s] && key[s] >= t));
            if (cnt >= K) {
                T = t;
                if (cnt == K) break;
            }
        }
        int gt = 0;
#pragma unroll
        for (int s = 0; s < KPL; ++s) gt += __popcll(__ballot(ok[s] && key[s] > T));
        int need = K - gt;  // ties at T: lowest candidate positions win
        int eq_before = 0, out_before = 0;
#pragma unroll
        for (int s = 0; s < KPL; ++s) {
            bool eq = ok[s] && key[s] == T;
            unsigned long long beq = __ballot(eq);
            bool take = (ok[s] && key[s] > T) || (eq && eq_before + __popcll(beq & below) < need);
            unsigned long long bt = __ballot(take);
            if (take) {
                const int pos = out_before + __popcll(bt & below);
                const int blk = cand ? cand[s * 64 + lane] : s * 64 + lane;
                orow[pos] = blk;
                if (lout) lout[r * Kq + pos] = blk;
                if (pc) atomicAdd(pc + s * 64 + lane, 1);
            }
            eq_before += __popcll(beq);
            out_before += __popcll(bt);
        }
    }
}

template <int KPL, int D>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ qbar,
                                                     const float* __restrict__ kbar,
                                                     const int* __restrict__ parent,
                                                     int* __restrict__ idx, Counts cnt,
                                                     int n_l, int K, int R, int M, float scale,
                                                     int causal)
{
    extern __shared__ float smem[];
    float* qs = smem;                 // [R][D]
    float* sc = qs + R * D;           // [R][M]
    int* cand = (int*)(sc + R * M);   // [M]
    int* pc = cand + M;               // [M] picks per candidate

    const int np = (n_l + BS - 1) / BS;  // parent-level blocks
    const int groups_per_head = parent ? np : (n_l + R - 1) / R;
    const int gh = blockIdx.x / groups_per_head;
    const int grp = blockIdx.x % groups_per_head;
    const int row0 = grp * (parent ? BS : R);
    const int rows = min(parent ? BS : R, n_l - row0);

    // candidate list (ascending)
    for (int c = threadIdx.x; c < M; c += blockDim.x) {
        if (parent) {
            const int* pr = parent + ((long)gh * np + grp) * (M / BS);  // parent row: M/16 picks
            cand[c] = child_of(pr[c / BS], c, np);  // may lie past n_l
        } else {
            cand[c] = c;
        }
        pc[c] = 0;
    }
    for (int e = threadIdx.x; e < rows * D; e += blockDim.x)
        qs[e] = qbar[((long)gh * n_l + row0) * D + e];
    __syncthreads();

    // score tile: four adjacent threads per candidate, D/4 channels each, so a
    // wave reads 16 whole candidate rows per load; the four partial dot
    // products are summed within the quad (DPP), identically in all four.
    constexpr int NV = D / 16;  // float4 per thread and row
    const int sub = threadIdx.x & 3;
    for (int c0 = 0; c0 < M; c0 += 64) {
        const int c = c0 + (threadIdx.x >> 2);
        const bool ok = c < M && cand[min(c, M - 1)] < n_l;  // children that exist
        float4 kv[NV];
        if (ok) {
            const float4* kr = (const float4*)(kbar + ((long)gh * n_l + cand[c]) * D + (D / 4) * sub);
#pragma unroll
            for (int t = 0; t < NV; ++t) kv[t] = kr[t];
        } else {
#pragma unroll
            for (int t = 0; t < NV; ++t) kv[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int r = 0; r < rows; ++r) {
            const float4* qr = (const float4*)(qs + r * D + (D / 4) * sub);
            float a = 0.f;
#pragma unroll
            for (int t = 0; t < NV; ++t) {
                const float4 qv = qr[t];
                a = fmaf(qv.x, kv[t].x, a);
                a = fmaf(qv.y, kv[t].y, a);
                a = fmaf(qv.z, kv[t].z, a);
                a = fmaf(qv.w, kv[t].w, a);
            }
            a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false));
            a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false));
            if (sub == 0 && c < M)  // + 0 turns -0 into +0; no child: never chosen
                sc[r * M + c] = ok ? causal_score(a * scale + 0.0f, cand[c], causal ? row0 + r : -1)
                                   : -INFINITY;
        }
    }
    __syncthreads();

    select_rows<KPL>(sc, cand, idx + ((long)gh * n_l + row0) * K, rows, M, K, pc);
    __syncthreads();
    flush_counts(pc, cand, M, {cnt.c1 + (long)gh * n_l, cnt.c16 + (long)gh * ((n_l + 15) / 16)});
}

// Sum of x over the 16 lanes of each DPP row (every lane gets its row's sum).
__device__ __forceinline__ int row16_sum(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);  // row_ror 4
    x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror 8
    return x;
}

// Top-K of 16 score rows (LDS, [16][M]; rows >= `rows` ignored), written in
// ascending candidate order to out[r * K ..].  Wave w takes rows 4w .. 4w+3,
// one per 16-lane group; lane n of a group holds the keys of candidates
// 16s + n (s < KPG), so all counting runs on the vector ALU with DPP row sums
// and the four rows of a wave advance together.
template <int KPG>
__device__ __forceinline__ void select_rows16(const float* sc, const int* cand, int* out,
                                              int rows, int M, int Kq, int* pc)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int r = 4 * wv + g;
    const bool live = r < rows;
    unsigned key[KPG];
    int nvalid = 0;
#pragma unroll
    for (int s = 0; s < KPG; ++s) {
        const int c = BS * s + n;
        // invalid candidates get key 0, below every finite score's key
        key[s] = (live && c < M) ? order_key(sc[r * M + c]) : 0u;
        nvalid += key[s] > KEY_NONE ? 1 : 0;
    }
    // the picks this row can make (K, but for a causal row with fewer
    // candidates); -1 in the slots after them
    const int K = min(Kq, row16_sum(nvalid));
    int* orow = out + (long)r * Kq;
    if (live)
        for (int p = K + n; p < Kq; p += 16) orow[p] = -1;
    // per-row threshold search, stopped per row as soon as exactly K keys
    // are >= T (see select_rows)
    unsigned T = 0;
    bool done = !live;
    for (int bit = 31; bit >= 0; --bit) {
        const unsigned t = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int s = 0; s < KPG; ++s) cnt += key[s] >= t ? 1 : 0;
        cnt = row16_sum(cnt);
        if (!done && cnt >= K) {
            T = t;
            done = cnt == K;
        }
        if (__all(done)) break;
    }
    int gt = 0;
#pragma unroll
    for (int s = 0; s < KPG; ++s) gt += key[s] > T ? 1 : 0;
    const int need = K - row16_sum(gt);  // ties at T: lowest candidate positions win
    const unsigned below = (1u << n) - 1u;
    const int sh = 16 * (g & 1);
    int eq_before = 0, out_before = 0;
#pragma unroll
    for (int s = 0; s < KPG; ++s) {
        const bool eq = live && key[s] == T;
        const unsigned long long beq = __ballot(eq);
        const unsigned meq = ((unsigned)(g < 2 ? beq : beq >> 32) >> sh) & 0xFFFFu;
        const bool take = (live && key[s] > T) || (eq && eq_before + __popc(meq & below) < need);
        const unsigned long long bt = __ballot(take);
        const unsigned mt = ((unsigned)(g < 2 ? bt : bt >> 32) >> sh) & 0xFFFFu;
        if (take) {
            orow[out_before + __popc(mt & below)] = cand[BS * s + n];
            atomicAdd(pc + BS * s + n, 1);
        }
        eq_before += __popc(meq);
        out_before += __popc(mt);
    }
}

// Query operand of the fp32 matrix-core scores: lane (g = lane/16, n =
// lane%16) holds channels (d/4)g .. (d/4)(g+1) - 1 of query row row0 + n
// (the last valid row repeated past `rows`).
template <int D>
__device__ __forceinline__ void load_query_operand(float (&qa)[D / 4], const float* qbar, long row0,
                                                   int rows)
{
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    constexpr int CG = D / 4;
    const float4* qr = (const float4*)(qbar + (row0 + min(n, rows - 1)) * D + CG * g);
#pragma unroll
    for (int t = 0; t < CG / 4; ++t) {
        const float4 v = qr[t];
        qa[4 * t] = v.x; qa[4 * t + 1] = v.y; qa[4 * t + 2] = v.z; qa[4 * t + 3] = v.w;
    }
}

// Scores on the fp32 matrix cores (v_mfma_f32_16x16x4_f32): 16 query rows x
// 16 candidates per tile; lane (g = lane/16, n = lane%16) feeds row n and
// candidate n over channels (d/4)g .. (d/4)(g+1) - 1, one channel per MFMA
// k-slot, so every lane reads whole 64-byte pieces of the rows.  The channel sum order is
// fixed by the instruction sequence.  Then the top-K of the `rows` rows
// (select_rows16) and the pick counts.  On entry cand and pc (LDS, M each)
// are filled and zeroed and a barrier has passed; kh = the head's key rows;
// crow0: the level row of output row 0 when causal, else -1.
template <int KPG, int D>
__device__ __forceinline__ void score_select16(const float (&qa)[D / 4], const float* kh, int* out,
                                               int rows, int M, int K, float scale, float* sc,
                                               const int* cand, int* pc, Counts cnt, int n_l,
                                               int crow0)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    constexpr int CG = D / 4;  // channels of lane group g: CG g .. CG g + CG - 1
    const int tiles = (M + BS - 1) / BS;
    kh += CG * g;
    auto load_tile = [&](float (&kb)[CG], int tile) {
        const int c = min(cand[min(tile * BS + n, M - 1)], n_l - 1);
        const float4* kr = (const float4*)(kh + (long)c * D);
#pragma unroll
        for (int t = 0; t < CG / 4; ++t) {
            const float4 v = kr[t];
            kb[4 * t] = v.x; kb[4 * t + 1] = v.y; kb[4 * t + 2] = v.z; kb[4 * t + 3] = v.w;
        }
    };
    float kb[CG], kn[CG];
    load_tile(kb, min(wv, tiles - 1));
    for (int tile = wv; tile < tiles; tile += 4) {
        load_tile(kn, min(tile + 4, tiles - 1));
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < CG; ++k)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[k], kb[k], acc, 0, 0, 0);
        const int col = tile * BS + n;
        // candidates past the level's last block (children the partial last
        // parent does not have) score -inf: never chosen
        const int cj = cand[min(col, M - 1)];
        const bool exists = col < M && cj < n_l;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r < rows && col < M)
                sc[(4 * g + r) * M + col] =
                    exists ? causal_score(acc[r] * scale + 0.0f, cj, crow0 < 0 ? -1 : crow0 + 4 * g + r)
                           : -INFINITY;
#pragma unroll
        for (int k = 0; k < CG; ++k) kb[k] = kn[k];
    }
    __syncthreads();
    select_rows16<KPG>(sc, cand, out, rows, M, K, pc);
    __syncthreads();
    flush_counts(pc, cand, M, cnt);
}

// Used for candidate lists of up to 1024.
template <int KPG, int D>
__global__ __launch_bounds__(256) void select_mfma(const float* __restrict__ qbar,
                                                   const float* __restrict__ kbar,
                                                   const int* __restrict__ parent,
                                                   int* __restrict__ idx, Counts cnt,
                                                   int n_l, int K, int M, float scale, int causal)
{
    extern __shared__ float smem[];
    float* sc = smem;                 // [16][M]
    int* cand = (int*)(sc + BS * M);  // [M]
    int* pc = cand + M;               // [M] picks per candidate
    // R rows per workgroup: the 16 siblings of a parent (they share their
    // candidates), or 4 rows of the coarsest level (more workgroups)
    const int R = parent ? BS : 4;
    const int groups_per_head = (n_l + R - 1) / R;
    const int gh = blockIdx.x / groups_per_head;
    const int grp = blockIdx.x % groups_per_head;
    const int row0 = grp * R;
    const int rows = min(R, n_l - row0);
    const int np = (n_l + BS - 1) / BS;  // parent-level blocks
    for (int c = threadIdx.x; c < M; c += blockDim.x) {
        if (parent) {
            const int* pr = parent + ((long)gh * np + grp) * (M / BS);  // parent row: M/16 picks
            cand[c] = child_of(pr[c / BS], c, np);  // may lie past n_l
        } else {
            cand[c] = c;
        }
        pc[c] = 0;
    }
    float qa[D / 4];
    load_query_operand<D>(qa, qbar, (long)gh * n_l + row0, rows);
    __syncthreads();
    score_select16<KPG, D>(qa, kbar + (long)gh * n_l * D, idx + ((long)gh * n_l + row0) * K, rows,
                           M, K, scale, sc, cand, pc,
                           {cnt.c1 + (long)gh * n_l, cnt.c16 + (long)gh * ((n_l + 15) / 16)}, n_l,
                           causal ? row0 : -1);
}

// The two coarsest levels in one launch.  Workgroup p (of a head) first
// chooses the top K_L of level-L row p among all n_L blocks, then -- with
// those picks kept in LDS as its candidate list -- the top K_{L-1} of the 16
// level-(L-1) rows 16p .. 16p+15 (the children of row p) exactly as
// select_mfma does.  Row p's scores are fp32 dot products, eight lanes per
// candidate (fixed order: each lane's channels in turn, then the lane sums
// pairwise); its top K_L is taken by one wave (select_rows).  Saves the coarsest level's launch and its write /
// read of the picks.  The coarsest level's picks are not counted (its
// transpose counts them itself): one count per workgroup and pick would put
// every workgroup's atomics on the same few addresses.  n_L <= 64 KPL.
// The body of select_top2 for coarsest row p of head gh; smem: the dynamic
// LDS of the launch, (16 M + 2 M + nL + Ktop) words.
template <int KPL, int KPG, int D>
__device__ __forceinline__ void top2_rows(const float* __restrict__ qtop,
                                          const float* __restrict__ ktop,
                                          const float* __restrict__ qbar,
                                          const float* __restrict__ kbar,
                                          int* __restrict__ idx_top, int* __restrict__ idx,
                                          Counts cnt, int nL, int n_l, int Ktop, int K,
                                          float scale, float* smem, int gh, int p, int causal)
{
    const int M = BS * Ktop;          // candidates of a level-(L-1) row
    float* sc = smem;                 // [16][M]
    int* cand = (int*)(sc + BS * M);  // [M]
    int* pc = cand + M;               // [M]
    float* st = (float*)(pc + M);     // [nL] scores of row p
    int* picks = (int*)(st + nL);     // [Ktop]
    for (int c = threadIdx.x; c < M; c += blockDim.x) pc[c] = 0;
    // row p's scores: eight lanes per candidate, lane u reading 16-byte
    // pieces u, u + 8, ... of the rows (query row p and key rows), so each
    // load instruction takes whole 128-byte lines of 8 key rows; PA rows per
    // lane group are loaded before the first is used
    constexpr int NT = D / 32;               // 16-byte pieces per lane and row
    constexpr int PA = D == D64 ? 4 : 2;     // rows in flight per lane group
    const int u = threadIdx.x & 7, rg = threadIdx.x >> 3;  // 32 lane groups
    float4 qv[NT];
    const float4* qrow = (const float4*)(qtop + ((long)gh * nL + p) * D);
#pragma unroll
    for (int t = 0; t < NT; ++t) qv[t] = qrow[u + 8 * t];
    const float* kt = ktop + (long)gh * nL * D;
    for (int c0 = 0; c0 < nL; c0 += 32 * PA) {
        float4 kv[PA][NT];
#pragma unroll
        for (int a = 0; a < PA; ++a) {
            const int c = min(c0 + 32 * a + rg, nL - 1);
#pragma unroll
            for (int t = 0; t < NT; ++t) kv[a][t] = ((const float4*)(kt + (long)c * D))[u + 8 * t];
        }
#pragma unroll
        for (int a = 0; a < PA; ++a) {
            float x = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                x = fmaf(qv[t].x, kv[a][t].x, x);
                x = fmaf(qv[t].y, kv[a][t].y, x);
                x = fmaf(qv[t].z, kv[a][t].z, x);
                x = fmaf(qv[t].w, kv[a][t].w, x);
            }
            // sum over the 8 lanes: within quads, then the two quads (half-row mirror)
            x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
            x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
            x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
            const int c = c0 + 32 * a + rg;
            if (u == 0 && c < nL)  // + 0 turns -0 into +0
                st[c] = causal_score(x * scale + 0.0f, c, causal ? p : -1);
        }
    }
    __syncthreads();
    if (threadIdx.x < 64)
        select_rows<KPL>(st, nullptr, idx_top + ((long)gh * nL + p) * Ktop, 1, nL, Ktop, nullptr,
                         picks);
    __syncthreads();
    // the children's query operand (loaded only now: phase-A registers are
    // free again, and its latency overlaps the first key tile's)
    // the children rows 16p .. (fewer under the partial last block)
    const int rows = min(BS, n_l - BS * p);
    float qa[D / 4];
    load_query_operand<D>(qa, qbar, (long)gh * n_l + BS * p, rows);
    for (int c = threadIdx.x; c < M; c += blockDim.x) cand[c] = child_of(picks[c / BS], c, nL);
    __syncthreads();
    score_select16<KPG, D>(qa, kbar + (long)gh * n_l * D, idx + ((long)gh * n_l + BS * p) * K,
                           rows, M, K, scale, sc, cand, pc,
                           {cnt.c1 + (long)gh * n_l, cnt.c16 + (long)gh * ((n_l + 15) / 16)}, n_l,
                           causal ? BS * p : -1);
}

template <int KPL, int KPG, int D>
__global__ __launch_bounds__(256) void select_top2(const float* __restrict__ qtop,
                                                   const float* __restrict__ ktop,
                                                   const float* __restrict__ qbar,
                                                   const float* __restrict__ kbar,
                                                   int* __restrict__ idx_top,
                                                   int* __restrict__ idx, Counts cnt,
                                                   int nL, int n_l, int Ktop, int K,
                                                   float scale, int causal)
{
    extern __shared__ float smem[];
    top2_rows<KPL, KPG, D>(qtop, ktop, qbar, kbar, idx_top, idx, cnt, nL, n_l, Ktop, K, scale,
                           smem, blockIdx.x / nL, blockIdx.x % nL, causal);
}

template <int KPG, int D>
hipError_t launch_mfma(const float* qbar, const float* kbar, const int* parent, int* idx,
                       Counts cnt, int G, int n_l, int K, int M, float scale, int causal,
                       hipStream_t st)
{
    const int groups = (n_l + (parent ? BS : 4) - 1) / (parent ? BS : 4);
    const size_t lds = (size_t)BS * M * sizeof(float) + 2 * (size_t)M * sizeof(int);
    if (lds > 65536) {  // 16 rows x 1024 candidates
        hipError_t e = hipFuncSetAttribute((const void*)select_mfma<KPG, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((select_mfma<KPG, D>), dim3(G * groups), dim3(256), lds, st, qbar, kbar, parent,
                       idx, cnt, n_l, K, M, scale, causal);
    return hipGetLastError();
}

template <int KPL, int KPG, int D>
hipError_t launch_top2(const Geo& g, const Ws& w, hipStream_t st)
{
    const int L = g.L, nL = g.n[L];
    const int M = BS * g.Kl[L];
    const size_t lds = (size_t)(BS * M + 2 * M + nL + g.Kl[L]) * sizeof(float);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)select_top2<KPL, KPG, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((select_top2<KPL, KPG, D>), dim3(g.G * nL), dim3(256), lds, st,
                       w.qbar[L - 1], w.kbar[L - 1], w.qbar[L - 2], w.kbar[L - 2], w.idx[L - 1],
                       w.idx[L - 2], Counts{w.cnt[L - 2], w.c16[L - 2]}, nL, g.n[L - 1],
                       g.Kl[L], g.Kl[L - 1], g.scale, (int)g.causal);
    return hipGetLastError();
}

template <int KPL, int D>
hipError_t launch_top2_k(const Geo& g, const Ws& w, hipStream_t st)
{
    const int M = BS * g.Kl[g.L];
    auto f = M <= 16 ? launch_top2<KPL, 1, D> : M <= 32 ? launch_top2<KPL, 2, D>
           : M <= 64 ? launch_top2<KPL, 4, D> : M <= 128 ? launch_top2<KPL, 8, D>
           : M <= 256 ? launch_top2<KPL, 16, D> : M <= 512 ? launch_top2<KPL, 32, D>
           : launch_top2<KPL, 64, D>;
    return f(g, w, st);
}

// Coarsest level with more than 1024 blocks: few rows per workgroup, so that
// the dense n_L x n_L scoring spreads over many CUs.
template <int KPL, int D>
hipError_t launch_wide(const float* qbar, const float* kbar, int* idx, Counts cnt, int G, int n_l,
                       int K, float scale, int causal, hipStream_t st)
{
    const int M = n_l;
    int R = max(1, min(min(16, n_l / 64), 8192 / M));
    int groups = (n_l + R - 1) / R;
    size_t lds = (size_t)(R * D + R * M) * sizeof(float) + 2 * (size_t)M * sizeof(int);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)select_kernel<KPL, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((select_kernel<KPL, D>), dim3(G * groups), dim3(256), lds, st, qbar, kbar,
                       nullptr, idx, cnt, n_l, K, R, M, scale, causal);
    return hipGetLastError();
}

template <int D>
hipError_t launch_select_d(const Geo& g, const Ws& w, bool zero_counts, hipStream_t st)
{
    if (zero_counts) {
        const unsigned cgrid = (unsigned)min((w.cnt_len + 255) / 256, 1024L);
        hipLaunchKernelGGL(clear_counts, dim3(cgrid), dim3(256), 0, st, w.cnt_all, w.cnt_len);
    }
    int l = g.L;
    // levels L and L-1 together when both fit the matrix-core path
    if (g.L >= 2 && g.n[g.L] <= 1024 && BS * g.Kl[g.L] <= 1024) {
        hipError_t e = g.n[g.L] <= 256 ? launch_top2_k<4, D>(g, w, st)
                                       : launch_top2_k<16, D>(g, w, st);
        if (e != hipSuccess) return e;
        l = g.L - 2;
    }
    for (; l >= 1; --l) {
        const int* parent = (l == g.L) ? nullptr : w.idx[l];
        const int K = g.Kl[l];  // picks of a level-l row
        const int M = parent ? BS * g.Kl[l + 1] : g.n[l];  // its candidates
        const float* qb = w.qbar[l - 1];
        const float* kb = w.kbar[l - 1];
        int* out = w.idx[l - 1];
        const Counts cnt = parent ? Counts{w.cnt[l - 1], w.c16[l - 1]} : Counts{nullptr, nullptr};
        hipError_t e;
        if (M <= 1024) {
            auto f = M <= 16 ? launch_mfma<1, D> : M <= 32 ? launch_mfma<2, D>
                   : M <= 64 ? launch_mfma<4, D> : M <= 128 ? launch_mfma<8, D>
                   : M <= 256 ? launch_mfma<16, D> : M <= 512 ? launch_mfma<32, D>
                   : launch_mfma<64, D>;
            e = f(qb, kb, parent, out, cnt, g.G, g.n[l], K, M, g.scale, (int)g.causal, st);
        } else {
            auto f = M <= 2048 ? launch_wide<32, D> : launch_wide<64, D>;
            e = f(qb, kb, out, cnt, g.G, g.n[l], K, g.scale, (int)g.causal, st);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_select(const Geo& g, const Ws& w, bool zero_counts, hipStream_t st)
{
    return g.d == D128 ? launch_select_d<D128>(g, w, zero_counts, st)
                       : launch_select_d<D64>(g, w, zero_counts, st);
}

}  // namespace llsa
