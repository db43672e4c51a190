// common.h -- internal definitions shared by the gfx950 kernels of libllsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llsa.h"

namespace llsa {

constexpr int BS = 16;      // block size (tokens per level-1 block)
constexpr int D64 = 64;     // head dimensions supported by the kernels: 64 and 128
constexpr int D128 = 128;
constexpr int MAX_L = LLSA_MAX_LEVELS;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

// Problem geometry derived once on the host and passed by value to kernels.
struct Geo {
    int G;                 // B * H
    int N;                 // tokens per head
    int K;                 // top-k of level 1 (the fine blocks), == Kl[1]
    int L;                 // pooling levels
    int n[MAX_L + 1];      // n[l] = ceil(N / 16^l) blocks at level l (n[0] = N); N is a
                           // multiple of 16, and the last block of a level l >= 2
                           // covers the tokens that remain (fewer than 16^l when
                           // 16^l does not divide N)
    int d;                 // head dimension (64 or 128)
    int Kl[MAX_L + 2];     // Kl[l]: picks per level-l row, l = 1..L
    // pooled entries of a query block: those of level l (l0 <= l <= L) are
    // entries eoff[l] .. eoff[l + 1] - 1; eoff[l0] = 0
    int eoff[MAX_L + 2];
    float scale;           // 1 / sqrt(d)
    unsigned flags;
    int l0;                // first level whose pooled tokens enrich (L + 1: none)
    float lb2;             // logit bias of a level-l pooled token: l * lb2 (log2 units)
    int xcd_chunk;         // workgroups per XCD chunk of the attention launches (xcd_block)
    bool cmp;              // LLSA_ENRICH_COMPLEMENT: the unpicked candidates enrich
    bool causal;           // LLSA_CAUSAL: token t attends keys u <= t
    // pooled entries per query block: the picks of the enriching levels (their
    // number), or with the complement at most the candidates of those levels
    __host__ __device__ int n_pooled() const { return l0 <= L ? eoff[L + 1] : 0; }
    __host__ __device__ int max_pooled() const
    {
        if (!cmp || l0 > L) return n_pooled();
        int m = 0;
        for (int l = l0; l <= L; ++l) m += l == L ? n[L] : BS * Kl[l + 1];
        return m;
    }
    // tokens covered by block j of level l (16^l but for a partial last block)
    __host__ __device__ int tokens(int l, int j) const
    {
        const long span = 1l << (4 * l), rest = (long)N - (long)j * span;
        return (int)(rest < span ? rest : span);
    }
    // level of pooled entry e (0 <= e < n_pooled())
    __host__ __device__ int entry_level(int e) const
    {
        int l = l0;
        while (l < L && e >= eoff[l + 1]) ++l;
        return l;
    }
};

// Device pointers into the caller's workspace.
struct Ws {
    float* qbar[MAX_L];
    float* kbar[MAX_L];
    float* vbar[MAX_L];
    int* idx[MAX_L];
    int* rowptr[MAX_L];
    int* col[MAX_L];
    unsigned char* slot[MAX_L];  // position of j in idx_l[col[e]] for each CSR entry e
    int* cnt[MAX_L];         // [G][n_l]: how many query blocks chose key block j
                             // (cleared and filled by select); feeds the transpose
    int* c16[MAX_L];         // [G][ceil(n_l/16)]: the same summed over 16 blocks
    int* cnt_all;            // all levels' cnt arrays, contiguous
    long cnt_len;            // their total length
    unsigned short* kb16;    // bf16 copies of kbar / vbar, all levels in one array:
    unsigned short* vb16;    //   row (prow[l] + gh * n_l + j) holds level l, head gh, block j
    long prow[MAX_L];        // first row of each level in kb16 / vb16
    float* delta;            // [G][N]
    float* pe1;              // [G][n1][K][2][16] bf16: P and dS of the level-1 pooled
                             // entries (the complement uses the region as fp32 partials)
    float* part[MAX_L];      // level l>=2 partial enrichment grads [G][n2][K][2][d]
    float* dbar[MAX_L];      // level l>=2 enrichment grads [G][n_l][2][d]
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf2f(unsigned short u)
{
    return __uint_as_float(((unsigned)u) << 16);
}

__device__ __forceinline__ unsigned short f2bf(float f)
{
    bf16 b = (bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(unsigned short, b);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float get(const float* p, long i) { return p[i]; }
};
template <> struct Elem<unsigned short> {
    static __device__ __forceinline__ float get(const unsigned short* p, long i) { return bf2f(p[i]); }
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS transposed read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j receives element (j & 3) of the 8-byte words read by lanes
// 4r + (j >> 2), r = 0..3.  So if lane 4r + x of a group reads row r,
// columns c0 + 4x .. c0 + 4x + 3 of a row-major bf16 matrix, lane j gets
// column c0 + j of rows 0..3: a column slice, i.e. the transposed operand.
__device__ __forceinline__ bf16x4 lds_read_tr(const void* lds_byte_ptr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(__attribute__((address_space(3))) char*)(lds_byte_ptr));
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Max / sum over the four lanes n, n+16, n+32, n+48 (one query row of an
// S^T tile): gfx950 v_permlane16_swap / v_permlane32_swap leave each lane
// holding its own value and its partner's, in some order; the result is the
// same in all four lanes (max is exact, a + b == b + a).
__device__ __forceinline__ float max_x4(float x)
{
    unsigned u = __float_as_uint(x);
    auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_x4(float x)
{
    unsigned u = __float_as_uint(x);
    auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Make all LDS writes of this wave visible to its later LDS reads, and keep
// the compiler from moving memory accesses across this point.
// Buffer loads: a resource per tensor (or per head) in scalar registers; the
// per-lane byte offset is loop-invariant and the row offset a scalar, so a
// gathered 16-row tile costs no vector address arithmetic.  Out-of-range
// offsets read zeros (hardware range check against num_bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned num_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}

__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ float bloadf(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// A row read once in the whole pass and not by the kernels that follow
// (a key block's own K and V rows in the dk/dv pass, O in the dq pass): a
// nontemporal load, so these rows do not displace the gathered tiles that
// other waves re-read from the caches (256x256: dk/dv 188 -> 178 us, dq
// 138 -> 135 us).
__device__ __forceinline__ bf16x8 ld8_once(const unsigned short* p)
{
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u16x8*)p));
}

// one bf16 element, widened to float (out of range: 0)
__device__ __forceinline__ float bload_bf16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0) << 16);
}

// A per-lane buffer offset that is out of range for any resource here: the
// load returns 0 (used to switch a lane's load off without a branch).
constexpr int OFF_NONE = 0x7ffffff0;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave: DPP sums within each 16-lane row, the
// four rows through permlane swaps, and lane 0's total broadcast so that
// every lane holds the identical value.
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm 1,0,3,2
    x += dpp_f<0x4E>(x);   // quad_perm 2,3,0,1
    x += dpp_f<0x124>(x);  // row_ror 4
    x += dpp_f<0x128>(x);  // row_ror 8
    x = sum_x4(x);
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ void lds_fence()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// An index read from the workspace (a block number, a list position or a
// slot), forced into [0, n) before it forms an address.  The backward and the
// single stages trust the workspace to hold what the forward of the same
// shape, top-k and flags wrote there; with any other contents the results
// are wrong, but every access stays inside the buffers the call was given.
__device__ __forceinline__ int clampi(int x, int n)
{
    return (int)min((unsigned)x, (unsigned)(n - 1));
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  Renumber them so that consecutive logical workgroups -- which
// work on neighbouring query or key blocks and gather the same candidate
// blocks -- run on the same XCD and share its L2: the r-th workgroup an XCD
// receives takes logical index (r / S) 8S + xcd S + r % S, i.e. the eight
// XCDs work through eight neighbouring chunks of S workgroups at a time.
// S = 0 means S = nb / 8: each XCD owns one contiguous eighth of the launch.
// A small S (Geo::xcd_chunk, chosen on the host) keeps the launch's front
// narrow, so that the tensors the workgroups in flight gather stay within the
// 256 MB MALL.  Workgroups past the last full round of 8S keep their index.
__device__ __forceinline__ int xcd_block(int b, int nb, int S)
{
    if (S <= 0) S = nb >> 3;
    if (S == 0) return b;
    const int span = 8 * S;
    const int full = nb / span * span;
    if (b >= full) return b;
    const int r = b >> 3;
    return (r / S) * span + (b & 7) * S + r % S;
}

// A 16-row bf16 tile of D channels loaded by one wave in 16-byte chunks: a
// row is D/8 chunks; one load instruction covers 1024 bytes (RPI rows), so a
// tile takes NI = D/32 loads per lane.  LDS row strides: ROW_T for tiles read
// back transposed (ds_read_b64_tr_b16), ROW_A for tiles read as MFMA operands;
// both shift successive rows by 8 or 4 banks, so the reads spread over all banks.
template <int D>
struct TileShape {
    static constexpr int LPR = D / 8;     // lanes per row
    static constexpr int RPI = 64 / LPR;  // rows per load instruction
    static constexpr int NI = BS / RPI;   // load instructions per tile
    static constexpr int ROW_T = D + 16;
    static constexpr int ROW_A = D + 8;
    static_assert(D == D64 || D == D128, "head dimension");
};

// Store a tile loaded as TileShape<D> chunks (load u: row lane/LPR + RPI u,
// columns 8 (lane % LPR) ..) into LDS rows of stride ROW.
template <int D, int ROW>
__device__ __forceinline__ void stage_rows(unsigned short* lds, const bf16x8 (&r)[TileShape<D>::NI],
                                           int lane)
{
    using TS = TileShape<D>;
    const int vr = lane / TS::LPR, vc = (lane % TS::LPR) * 8;
#pragma unroll
    for (int u = 0; u < TS::NI; ++u) *(bf16x8*)(lds + (vr + TS::RPI * u) * ROW + vc) = r[u];
}

// MFMA operand rows of a staged tile: row lane%16, channels 32u + 8(lane/16)
// .. +7 for u < D/32 (the A or B operand of a 16x16x32 product over D).
template <int D, int ROW>
__device__ __forceinline__ void operand_rows(const unsigned short* lds,
                                             bf16x8 (&x)[TileShape<D>::NI], int lane)
{
    const int gq = lane >> 4, nq = lane & 15;
#pragma unroll
    for (int u = 0; u < TileShape<D>::NI; ++u)
        x[u] = *(const bf16x8*)(lds + nq * ROW + 32 * u + 8 * gq);
}

// 16x16 product over D channels: D/32 chained 16x16x32 MFMAs
template <int D>
__device__ __forceinline__ f32x4 scores(const bf16x8 (&a)[TileShape<D>::NI],
                                        const bf16x8 (&b)[TileShape<D>::NI])
{
    f32x4 s = {};
#pragma unroll
    for (int u = 0; u < TileShape<D>::NI; ++u) s = mfma32(a[u], b[u], s);
    return s;
}

// An entry of a query block's pooled-entry table (LDS): the row of the
// pooled token in the bf16 pooled arrays, with its level in bits 28..30
// (rows stay below 2^28: B*H*N < 2^31 tokens give fewer than 2^27 blocks).
constexpr int ENT_ROW = (1 << 28) - 1;
__device__ __forceinline__ int ent_level(int e) { return e >> 28; }

// Fill the pooled-entry table of query block i (head gh) and return the
// number of entries (the same in every lane of the wave).  Default: the
// picks of its ancestor at every enriching level l0..L, level by level.
// LLSA_CAUSAL: of those only the picks before the ancestor itself (its own
// block's mean holds later tokens; unused slots hold -1), compacted by
// ballot -- the level-1 entries then keep the positions of their picks.
// LLSA_ENRICH_COMPLEMENT: at every enriching level the ancestor's candidates
// it did not pick -- all blocks at the coarsest level, below it the existing
// children of the parent's picks -- in ascending order, compacted by ballot.
__device__ __forceinline__ int fill_entries(const Geo& g, const Ws& w, int gh, int i, int* ent,
                                            int lane)
{
    int E = 0;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int l = g.l0; l <= g.L; ++l) {
        const int Kl = g.Kl[l], nl = g.n[l];
        const int a = i >> (4 * (l - 1));
        const int* sel = w.idx[l - 1] + ((long)gh * nl + a) * Kl;
        const long row0 = w.prow[l - 1] + (long)gh * nl;
        if (g.causal) {  // Kl <= 64: one pick per lane
            const int j = lane < Kl ? sel[lane] : -1;
            const bool keep = j >= 0 && j != a;
            const unsigned long long bal = __ballot(keep);
            if (keep) ent[E + __popcll(bal & below)] = (int)(row0 + clampi(j, nl)) | (l << 28);
            E += __popcll(bal);
            continue;
        }
        if (!g.cmp) {
            for (int s0 = 0; s0 < Kl; s0 += 64)
                if (s0 + lane < Kl)
                    ent[E + s0 + lane] = (int)(row0 + clampi(sel[s0 + lane], nl)) | (l << 28);
            E += Kl;
            continue;
        }
        // the ancestor's picks, one per lane (Kl <= 64)
        const int mine = lane < Kl ? clampi(sel[lane], nl) : -1;
        const int M = l == g.L ? nl : BS * g.Kl[l + 1];
        const int* par = l == g.L ? nullptr
                                  : w.idx[l] + ((long)gh * g.n[l + 1] + (a >> 4)) * g.Kl[l + 1];
        for (int c0 = 0; c0 < M; c0 += 64) {
            const int c = c0 + lane;
            int j = nl;
            if (c < M) j = par ? BS * clampi(par[c >> 4], g.n[l + 1]) + (c & 15) : c;
            bool keep = j < nl;  // past the level's last block: no such child
            for (int p = 0; p < Kl; ++p) keep = keep && j != __builtin_amdgcn_readlane(mine, p);
            const unsigned long long bal = __ballot(keep);
            if (keep) ent[E + __popcll(bal & below)] = (int)(row0 + j) | (l << 28);
            E += __popcll(bal);
        }
    }
    return E;
}

// Visit the pooled entries of query block i (head gh), level by level, in
// the order fill_entries lists them: f(level, block) (uniform in the wave;
// the fp32 kernels).
template <typename F>
__device__ __forceinline__ void for_each_pooled(const Geo& g, const Ws& w, int gh, int i, F f)
{
    for (int l = g.l0; l <= g.L; ++l) {
        const int Kl = g.Kl[l], nl = g.n[l];
        const int a = i >> (4 * (l - 1));
        const int* sel = w.idx[l - 1] + ((long)gh * nl + a) * Kl;
        if (!g.cmp) {
            for (int s = 0; s < Kl; ++s)
                if (!g.causal || (sel[s] >= 0 && sel[s] != a)) f(l, clampi(sel[s], nl));
            continue;
        }
        const int M = l == g.L ? nl : BS * g.Kl[l + 1];
        const int* par = l == g.L ? nullptr
                                  : w.idx[l] + ((long)gh * g.n[l + 1] + (a >> 4)) * g.Kl[l + 1];
        for (int c = 0; c < M; ++c) {
            const int j = par ? BS * clampi(par[c >> 4], g.n[l + 1]) + (c & 15) : c;
            if (j >= nl) continue;
            bool picked = false;
            for (int s = 0; s < Kl; ++s) picked = picked || sel[s] == j;
            if (!picked) f(l, j);
        }
    }
}

// ------------------------------------------------------------ fp32 row batches
//
// The fp32 kernels hold one row per wave (a token's query, a key, or a pooled
// token) and visit the rows it meets 16 at a time.  Lane layout: lane =
// r + 16 cg holds batch row r's channels CH cg .. CH cg + CH - 1 (CH = D/4)
// and the same slice of the wave's own row.  A dot product is CH fmas in the
// lane and a sum over the four channel groups (sum_x4, the same value in all
// four lanes of the row); a row-weighted sum of rows (o, dq, dk, dv, pooled
// gradients) accumulates per lane and is summed over the 16 rows once, at
// the end (row16_sum).  A batch's loads are all in flight together.
//
// A batch: lane r + 16 cg holds row r's key and value pointers and logit
// bias; rows at or past n hold row 0's (valid memory; the caller masks them).

struct RowBatch {
    const float* k;
    const float* v;
    float bias;
    int n;  // rows in the batch (wave-uniform)
};

// Collects rows one at a time and hands every full batch, and at finish()
// the last partial one, to `flush`.
template <typename F>
struct RowBatcher {
    RowBatch b;
    int row;  // lane % 16
    F& flush;
    __device__ RowBatcher(int lane, F& f) : b{nullptr, nullptr, 0.f, 0}, row(lane & 15), flush(f) {}
    __device__ void push(const float* k, const float* v, float bias)
    {
        if (b.n == 0 || row == b.n) {
            b.k = k;
            b.v = v;
            b.bias = bias;
        }
        if (++b.n == BS) {
            flush(b);
            b.n = 0;
        }
    }
    __device__ void finish()
    {
        if (b.n > 0) flush(b);
        b.n = 0;
    }
};

// channels D/4 cg .. D/4 cg + D/4 - 1 of a row (16-byte loads)
template <int D>
__device__ __forceinline__ void load_slice(float (&x)[D / 4], const float* row, int lane)
{
    const float4* p = (const float4*)(row + (D / 4) * (lane >> 4));
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
        const float4 t = p[u];
        x[4 * u] = t.x;
        x[4 * u + 1] = t.y;
        x[4 * u + 2] = t.z;
        x[4 * u + 3] = t.w;
    }
}

template <int D>
__device__ __forceinline__ float slice_dot(const float (&a)[D / 4], const float (&b)[D / 4])
{
    float part = a[0] * b[0];
#pragma unroll
    for (int c = 1; c < D / 4; ++c) part = fmaf(a[c], b[c], part);
    return sum_x4(part);
}

// Sum / max over the 16 lanes of each DPP row (every lane gets the result).
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm 1,0,3,2
    x += dpp_f<0x4E>(x);   // quad_perm 2,3,0,1
    x += dpp_f<0x124>(x);  // row_ror 4
    x += dpp_f<0x128>(x);  // row_ror 8
    return x;
}

__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x124>(x));
    x = fmaxf(x, dpp_f<0x128>(x));
    return x;
}

// A query token's key/value set as batches: each fine block of its level-1
// list (its 16 rows; under LLSA_CAUSAL unused slots skipped and the diagonal
// block cut to the keys at or before t), then the pooled tokens of the
// enriching levels (a level-lv token's logit gets lb2 * lv * ln 2).
template <int D, typename F>
__device__ __forceinline__ void for_each_batch(const Geo& g, const Ws& w, const float* k,
                                               const float* v, int gh, int t, int lane, F& run)
{
    const int* sel = w.idx[0] + ((long)gh * g.n[1] + t / BS) * g.K;
    for (int s = 0; s < g.K; ++s) {
        const int j = sel[s];
        if (g.causal && j < 0) continue;  // an unused slot
        const int cnt = (g.causal && j == t / BS) ? t % BS + 1 : BS;
        const long row =
            ((long)gh * g.N + (long)clampi(j, g.n[1]) * BS + min(lane & 15, cnt - 1)) * D;
        run(RowBatch{k + row, v + row, 0.f, cnt});
    }
    RowBatcher<F> bat(lane, run);
    for_each_pooled(g, w, gh, t / BS, [&](int lv, int j) {
        const long row = ((long)gh * g.n[lv] + j) * D;
        bat.push(w.kbar[lv - 1] + row, w.vbar[lv - 1] + row, g.lb2 * (float)lv * LN2);
    });
    bat.finish();
}

// ------------------------------------------------------------ grid order

__device__ __forceinline__ unsigned gather_bits(unsigned x)  // inverse of spread_bits
{
    x &= 0x55555555u;
    x = (x | (x >> 1)) & 0x33333333u;
    x = (x | (x >> 2)) & 0x0f0f0f0fu;
    x = (x | (x >> 4)) & 0x00ff00ffu;
    x = (x | (x >> 8)) & 0x0000ffffu;
    return x;
}

__device__ __forceinline__ unsigned gather3(unsigned x)  // inverse of spread3
{
    x &= 0x09249249u;
    x = (x | (x >> 2)) & 0x030c30c3u;
    x = (x | (x >> 4)) & 0x0300f00fu;
    x = (x | (x >> 8)) & 0xff0000ffu;
    x = (x | (x >> 16)) & 0x000003ffu;
    return x;
}

// Grid order of frames x height x width cells (LLSA README, reordering of
// non-sequential data, extended to rectangles and video): tiles of S x S
// (S^3 for video) cells in raster order, S the largest power of two dividing
// every side; Morton order inside a tile with the frame bit above the row bit
// above the column bit.  A square power-of-two image is one tile.
struct GridGeo {
    unsigned H, W;        // rows, columns
    unsigned tw, th;      // tiles per row, tile rows per frame slab
    int s_log2;           // log2 S
    int video;            // 3-D tiles
};


inline GridGeo make_grid_geo(int frames, int height, int width)
{
    auto p2 = [](int v) { return v & -v; };
    int S = p2(height) < p2(width) ? p2(height) : p2(width);
    const int video = frames > 1;
    if (video && p2(frames) < S) S = p2(frames);
    GridGeo gg;
    gg.H = (unsigned)height;
    gg.W = (unsigned)width;
    gg.tw = (unsigned)(width / S);
    gg.th = (unsigned)(height / S);
    gg.s_log2 = __builtin_ctz((unsigned)S);
    gg.video = video;
    return gg;
}

// The raster cell (frame, row, column flattened) of grid-order position p.
__device__ __forceinline__ unsigned grid_source(unsigned p, const GridGeo& gg)
{
    const int tb = (gg.video ? 3 : 2) * gg.s_log2;  // bits of a position inside a tile
    const unsigned code = p & ((1u << tb) - 1u), tile = p >> tb;
    unsigned yy, xx, tt = 0;
    if (gg.video) {
        xx = gather3(code);
        yy = gather3(code >> 1);
        tt = gather3(code >> 2);
    } else {
        xx = gather_bits(code);
        yy = gather_bits(code >> 1);
    }
    const unsigned tx = tile % gg.tw, rest = tile / gg.tw;
    const unsigned ty = rest % gg.th, tz = rest / gg.th;
    const unsigned y = (ty << gg.s_log2) | yy, x = (tx << gg.s_log2) | xx;
    const unsigned t = (tz << gg.s_log2) | tt;  // frame (0 for an image)
    return (t * gg.H + y) * gg.W + x;
}

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.

hipError_t launch_grid_order(const void* src, void* dst, long long outer, int frames, int height,
                             int width, int inner_bytes, int inverse, hipStream_t st);
hipError_t launch_zorder(const void* src, void* dst, long long outer, int side, int inner_bytes,
                         int inverse, hipStream_t st);
// zero_counts: pool zeroes the selection's pick counters (llsa_forward);
// select zeroes them itself (the selection part on its own)
hipError_t launch_pool(const void* q, const void* k, const void* v, int dtype, const Geo& g,
                       const Ws& w, bool zero_counts, hipStream_t st);
// the pool pass that also gathers raster-order q, k, v (qr, kr, vr) into q,
// k, v in grid order; zeroes the selection's pick counters like launch_pool
hipError_t launch_pool_gather(const void* qr, const void* kr, const void* vr, void* q, void* k,
                              void* v, const GridGeo& gg, int dtype, const Geo& g, const Ws& w,
                              hipStream_t st);
hipError_t launch_select(const Geo& g, const Ws& w, bool zero_counts, hipStream_t st);
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                           int dtype, const Geo& g, const Ws& w, hipStream_t st);
hipError_t launch_transpose(const Geo& g, const Ws& w, hipStream_t st);
// The first transpose launch: the two coarsest levels together (pair) when
// the coarsest level has at most 1024 blocks, else the coarsest alone -- its
// level argument, pair flag and workgroup count; and the launches of the
// levels it does not build.
struct TrFirst {
    int l, pair, wgs;
};
TrFirst transpose_first(const Geo& g);
hipError_t launch_transpose_after(const Geo& g, const Ws& w, const TrFirst& f, hipStream_t st);
// bf16 dQ with the first transpose launch's workgroups in front of its own
// (both read only the forward's results and write disjoint workspace
// regions), so the latency-bound transpose overlaps dQ in one launch.
hipError_t launch_attn_dq_transpose(const void* q, const void* k, const void* v, const void* out,
                                    const float* lse, const void* dout, void* dq, const Geo& g,
                                    const Ws& w, hipStream_t st);
hipError_t launch_attn_dq(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, void* dq, int dtype, const Geo& g,
                          const Ws& w, hipStream_t st);
hipError_t launch_attn_enrich(const void* q, const float* lse, const void* dout, int dtype,
                              const Geo& g, const Ws& w, hipStream_t st);
hipError_t launch_attn_dkdv(const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, void* dk, void* dv, int dtype, const Geo& g,
                            const Ws& w, hipStream_t st);

}  // namespace llsa
