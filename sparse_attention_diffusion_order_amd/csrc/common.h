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
    int n[MAX_L + 1];      // n[l] = N / 16^l blocks at level l (n[0] = N)
    int d;                 // head dimension (64 or 128)
    int Kl[MAX_L + 2];     // Kl[l]: picks per level-l row, l = 1..L
    // pooled entries of a query block: those of level l (l0 <= l <= L) are
    // entries eoff[l] .. eoff[l + 1] - 1; eoff[l0] = 0
    int eoff[MAX_L + 2];
    float scale;           // 1 / sqrt(d)
    unsigned flags;
    int l0;                // first level whose pooled tokens enrich (L + 1: none)
    float lb2;             // logit bias of a level-l pooled token: l * lb2 (log2 units)
    __host__ __device__ int n_pooled() const { return l0 <= L ? eoff[L + 1] : 0; }
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
    float* pe1;              // [G][n1][K][2][16]: P and dS of the level-1 pooled entries
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

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  Renumber them so that consecutive logical workgroups -- which
// work on neighbouring query or key blocks and gather the same candidate
// blocks -- run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_block(int b, int nb)
{
    const int full = nb & ~7;
    if (b >= full) return b;
    return (b & 7) * (full >> 3) + (b >> 3);
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
