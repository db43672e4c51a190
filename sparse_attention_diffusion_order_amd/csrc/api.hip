// api.hip -- C ABI of libllsa: validation, workspace layout and launch order.
//
// Every check happens before the first HIP call, so argument errors are
// reported identically on a host without a GPU.
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "common.h"

using namespace llsa;

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

// ks[l - 1]: picks per level-l row (l = 1..levels)
int validate(int B, int H, int N, int d, int block_size, const int* ks, int levels, int dtype,
             unsigned flags)
{
    if (!ks) return LLSA_ERR_NULL;
    if ((d != D64 && d != D128) || block_size != BS || (dtype != LLSA_F32 && dtype != LLSA_BF16) ||
        (flags & ~LLSA_KNOWN_FLAGS))
        return LLSA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || N < BS || levels < 1) return LLSA_ERR_SHAPE;
    if (levels > MAX_L) return LLSA_ERR_UNSUPPORTED;
    if (N % BS) return LLSA_ERR_SHAPE;  // whole level-1 blocks
    // level l has ceil(N / 16^l) blocks, the last one partial when 16^l does
    // not divide N
    long long n[MAX_L + 2];
    n[0] = N;
    for (int l = 1; l <= levels; ++l) n[l] = (n[l - 1] + BS - 1) / BS;
    const long long nL = n[levels];
    // level l chooses among the n_L blocks (coarsest) or the existing
    // children of its parent's K_{l+1} picks: at worst 16 (K_{l+1} - 1) full
    // parents and the last, partial one
    // (the same limit holds for causal rows, which keep fewer picks where
    // they have fewer earlier candidates: the workspace size depends on the
    // shape and top-k only)
    for (int l = levels; l >= 1; --l) {
        const long long cands =
            l == levels ? nL : (long long)BS * (ks[l] - 1) + (n[l] - BS * (n[l + 1] - 1));
        if (ks[l - 1] < 1 || ks[l - 1] > cands) return LLSA_ERR_SHAPE;
    }
    // the complement is defined for the non-causal selection only
    if ((flags & LLSA_CAUSAL) && (flags & LLSA_ENRICH_COMPLEMENT)) return LLSA_ERR_UNSUPPORTED;
    for (int l = 0; l < levels; ++l)
        if (ks[l] > 64) return LLSA_ERR_UNSUPPORTED;
    if (nL > 4096) return LLSA_ERR_UNSUPPORTED;
    if ((flags & LLSA_ENRICH_COMPLEMENT) && !(flags & LLSA_NO_ENRICH)) {
        // the complement's entries per query block: the candidates of the
        // enriching levels, at most 2048 (the entry table of the kernels)
        long long m = 0;
        for (int l = (flags & LLSA_ENRICH_COARSE) ? 2 : 1; l <= levels; ++l)
            m += l == levels ? nL : (long long)BS * ks[l];
        if (m > 2048) return LLSA_ERR_UNSUPPORTED;
    }
    if ((long long)B * H * N >= (1ll << 31)) return LLSA_ERR_UNSUPPORTED;
    if (N > (1 << 23)) return LLSA_ERR_UNSUPPORTED;  // one head's tensor < 2 GiB (buffer offsets)
    return LLSA_OK;
}

struct Layout {
    llsa_ws_layout pub;
    size_t kb16, vb16, pe1, cnt;
    size_t slot[MAX_L];
    size_t part[MAX_L];
    size_t dbar[MAX_L];
    bool fwd_only;  // only the forward's parts (no backward state)
};

// Workspace: pyramid (float32), index lists, key->query CSR lists, delta,
// enrichment gradient partials and sums.  Sizes are O(B*H*N*d): no part of
// it grows with the square of the block count.  fwd_only: the parts the
// forward uses (pyramid, index lists, bf16 pooled copies, pick counts).
void make_layout(int G, int N, int D, const int* ks, int L, Layout* lay, bool fwd_only = false)
{
    memset(lay, 0, sizeof(*lay));
    lay->fwd_only = fwd_only;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    long long n[MAX_L + 1];
    n[0] = N;
    for (int l = 1; l <= L; ++l) n[l] = (n[l - 1] + BS - 1) / BS;
    for (int l = 1; l <= L; ++l) {
        size_t pyr = (size_t)G * n[l] * D * sizeof(float);
        lay->pub.qbar[l - 1] = take(pyr);
        lay->pub.kbar[l - 1] = take(pyr);
        lay->pub.vbar[l - 1] = take(pyr);
        lay->pub.idx[l - 1] = take((size_t)G * n[l] * ks[l - 1] * sizeof(int));
    }
    for (int l = 1; l <= L && !fwd_only; ++l) {
        lay->pub.rowptr[l - 1] = take((size_t)G * (n[l] + 1) * sizeof(int));
        lay->pub.col[l - 1] = take((size_t)G * n[l] * ks[l - 1] * sizeof(int));
    }
    size_t prows = 0;
    for (int l = 1; l <= L; ++l) prows += (size_t)G * n[l];
    lay->kb16 = take(prows * D * 2);
    lay->vb16 = take(prows * D * 2);
    size_t blocks = 0;
    for (int l = 1; l <= L; ++l)
        blocks += (size_t)G * (n[l] + (n[l] + 15) / 16);
    lay->cnt = take(blocks * sizeof(int));
    if (fwd_only) {
        lay->pub.total = off;
        return;
    }
    lay->pub.delta = take((size_t)G * N * sizeof(float));
    lay->pe1 = take((size_t)G * n[1] * ks[0] * 2 * BS * sizeof(float));
    for (int l = 1; l <= L; ++l) lay->slot[l - 1] = take((size_t)G * n[l] * ks[l - 1]);
    for (int l = 1; l <= L; ++l) {
        lay->dbar[l - 1] = take((size_t)G * n[l] * 2 * D * sizeof(float));
        if (l >= 2) lay->part[l - 1] = take((size_t)G * n[2] * ks[l - 1] * 2 * D * sizeof(float));
    }
    lay->pub.total = off;
}

void make_geo(int B, int H, int N, int d, const int* ks, int levels, unsigned flags, int dtype,
              Geo* g)
{
    memset(g, 0, sizeof(*g));
    g->G = B * H;
    g->N = N;
    g->d = d;
    g->K = ks[0];
    g->L = levels;
    g->n[0] = N;
    for (int l = 1; l <= levels; ++l) {
        g->n[l] = (g->n[l - 1] + BS - 1) / BS;  // the last block may be partial
        g->Kl[l] = ks[l - 1];
    }
    g->scale = 1.0f / sqrtf((float)d);  // SDPA's default scale
    g->flags = flags;
    g->l0 = (flags & LLSA_NO_ENRICH) ? levels + 1 : (flags & LLSA_ENRICH_COARSE) ? 2 : 1;
    g->lb2 = (flags & LLSA_SIZE_BIAS) ? 4.0f : 0.0f;  // log2(16^l) = 4 l
    g->cmp = (flags & LLSA_ENRICH_COMPLEMENT) != 0;
    g->causal = (flags & LLSA_CAUSAL) != 0;
    // The attention launches gather key/value (forward, dQ) or query/dO
    // (dK/dV) rows of every head.  While those of all heads fit well inside
    // the 256 MB MALL, each XCD takes one contiguous eighth of the launch
    // (best L2 locality); beyond that the XCDs move together through chunks
    // of 256 workgroups so that the rows in flight stay in the MALL
    // (measured at 512x512, six heads: forward + backward 2.75 -> 2.54 ms;
    // at 256x256 the chunks cost 2.5 %).
    const double gathered = 2.0 * g->G * (double)N * d * (dtype == LLSA_BF16 ? 2 : 4);
    g->xcd_chunk = gathered > 192.0 * (1 << 20) ? 256 : 0;
    int e = 0;  // pooled entry offsets of the enriching levels
    for (int l = g->l0; l <= levels; ++l) {
        g->eoff[l] = e;
        e += ks[l - 1];
    }
    g->eoff[levels + 1] = e;
}

// Pointers into the workspace at `base` (the backward's parts stay null in a
// forward-only layout).
void make_ws(void* base, const Layout& lay, int L, Ws* w)
{
    memset(w, 0, sizeof(*w));
    char* b = (char*)base;
    const bool bwd = !lay.fwd_only;
    for (int l = 1; l <= L; ++l) {
        w->qbar[l - 1] = (float*)(b + lay.pub.qbar[l - 1]);
        w->kbar[l - 1] = (float*)(b + lay.pub.kbar[l - 1]);
        w->vbar[l - 1] = (float*)(b + lay.pub.vbar[l - 1]);
        w->idx[l - 1] = (int*)(b + lay.pub.idx[l - 1]);
        if (!bwd) continue;
        w->rowptr[l - 1] = (int*)(b + lay.pub.rowptr[l - 1]);
        w->col[l - 1] = (int*)(b + lay.pub.col[l - 1]);
        w->slot[l - 1] = (unsigned char*)(b + lay.slot[l - 1]);
        w->dbar[l - 1] = (float*)(b + lay.dbar[l - 1]);
        if (l >= 2) w->part[l - 1] = (float*)(b + lay.part[l - 1]);
    }
    if (bwd) {
        w->delta = (float*)(b + lay.pub.delta);
        w->pe1 = (float*)(b + lay.pe1);
    }
    w->cnt_all = (int*)(b + lay.cnt);
    w->kb16 = (unsigned short*)(b + lay.kb16);
    w->vb16 = (unsigned short*)(b + lay.vb16);
}

struct Prep {
    Geo geo;
    Ws ws;
    hipStream_t st;
};

// Tensor arguments: the kernels move rows of q, k, v, out, dout and the
// gradients (and workspace regions) in 16-byte pieces, lse in 4-byte ones.
bool bad16(const void* p) { return !p || ((uintptr_t)p & 15u); }

template <typename... P>
bool any_bad16(P... p)
{
    return (bad16(p) || ...);
}

bool bad_lse(const float* p) { return !p || ((uintptr_t)p & 3u); }

int prepare(int B, int H, int N, int d, int block_size, const int* ks, int levels, int dtype,
            unsigned flags, void* workspace, size_t ws_bytes, void* stream, Prep* p,
            bool fwd_only = false)
{
    int rc = validate(B, H, N, d, block_size, ks, levels, dtype, flags);
    if (rc) return rc;
    Layout lay;
    make_layout(B * H, N, d, ks, levels, &lay, fwd_only);
    if (bad16(workspace) || ws_bytes < lay.pub.total) return LLSA_ERR_WORKSPACE;
    make_geo(B, H, N, d, ks, levels, flags, dtype, &p->geo);
    make_ws(workspace, lay, levels, &p->ws);
    // per-level block rows of the bf16 pyramid copies; the choice counts
    // (per block and per 16 blocks) of every level
    long r = 0, c = 0;
    const long G = p->geo.G;
    for (int l = 1; l <= levels; ++l) {
        const long nl = p->geo.n[l];
        p->ws.prow[l - 1] = r;
        r += G * nl;
        p->ws.cnt[l - 1] = p->ws.cnt_all + c;
        c += G * nl;
        p->ws.c16[l - 1] = p->ws.cnt_all + c;
        c += G * ((nl + 15) / 16);
    }
    p->ws.cnt_len = c;
    p->st = (hipStream_t)stream;
    return LLSA_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? LLSA_OK : LLSA_ERR_HIP; }

int run_forward_part(int part, const void* q, const void* k, const void* v, void* out,
                     float* lse, int dtype, const Prep& p)
{
    switch (part) {
    case LLSA_PART_POOL: return hip_rc(launch_pool(q, k, v, dtype, p.geo, p.ws, false, p.st));
    case LLSA_PART_SELECT: return hip_rc(launch_select(p.geo, p.ws, true, p.st));
    case LLSA_PART_ATTN:
        return hip_rc(launch_attn_fwd(q, k, v, out, lse, dtype, p.geo, p.ws, p.st));
    default: return LLSA_ERR_UNSUPPORTED;
    }
}

// The whole forward.  The pool launch zeroes the pick counters the selection
// adds to (one launch fewer than the selection part on its own, which zeroes
// them itself).
int run_forward(const void* q, const void* k, const void* v, void* out, float* lse, int dtype,
                const Prep& p)
{
    int rc = hip_rc(launch_pool(q, k, v, dtype, p.geo, p.ws, true, p.st));
    if (rc) return rc;
    rc = hip_rc(launch_select(p.geo, p.ws, false, p.st));
    if (rc) return rc;
    return run_forward_part(LLSA_PART_ATTN, q, k, v, out, lse, dtype, p);
}

int run_backward_part(int part, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int dtype, const Prep& p)
{
    switch (part) {
    case LLSA_PART_TRANSPOSE: return hip_rc(launch_transpose(p.geo, p.ws, p.st));
    case LLSA_PART_DQ:
        return hip_rc(launch_attn_dq(q, k, v, out, lse, dout, dq, dtype, p.geo, p.ws, p.st));
    case LLSA_PART_ENRICH:
        return hip_rc(launch_attn_enrich(q, lse, dout, dtype, p.geo, p.ws, p.st));
    case LLSA_PART_DKDV:
        return hip_rc(launch_attn_dkdv(q, k, v, lse, dout, dk, dv, dtype, p.geo, p.ws, p.st));
    default: return LLSA_ERR_UNSUPPORTED;
    }
}

// The scratch of llsa_forward_noalloc: one array in each GPU's memory,
// reserved when the library's code object is loaded on that GPU and held
// until the process ends.  In host code `scratch` only names the array;
// its device address on the current GPU comes from hipGetSymbolAddress,
// looked up once per device and kept in noalloc_base.
static __device__ __align__(256) unsigned char scratch[LLSA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> noalloc_base[MAX_DEVICES];

// Device address of the current GPU's scratch (set up on the first call on
// that GPU, with it current).
int noalloc_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return LLSA_ERR_HIP;
    void* ptr = noalloc_base[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return LLSA_ERR_HIP;
        noalloc_base[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return LLSA_OK;
}

// the same top-k at every level, as an array (levels outside 1..MAX_L are
// rejected by validate before the array is read)
struct UniformK {
    int ks[MAX_L];
    UniformK(int topk, int levels)
    {
        for (int l = 0; l < MAX_L; ++l) ks[l] = l < levels ? topk : 0;
    }
};

}  // namespace

extern "C" {

size_t llsa_workspace_bytes_lk(int B, int H, int N, int d, int block_size, const int* topk,
                               int levels, int dtype)
{
    if (validate(B, H, N, d, block_size, topk, levels, dtype, 0)) return 0;
    Layout lay;
    make_layout(B * H, N, d, topk, levels, &lay);
    return lay.pub.total;
}

size_t llsa_workspace_bytes(int B, int H, int N, int d, int block_size, int topk, int levels,
                            int dtype)
{
    return llsa_workspace_bytes_lk(B, H, N, d, block_size, UniformK(topk, levels).ks, levels,
                                   dtype);
}

int llsa_workspace_layout_lk(int B, int H, int N, int d, int block_size, const int* topk,
                             int levels, int dtype, llsa_ws_layout* out)
{
    if (!out) return LLSA_ERR_NULL;
    int rc = validate(B, H, N, d, block_size, topk, levels, dtype, 0);
    if (rc) return rc;
    Layout lay;
    make_layout(B * H, N, d, topk, levels, &lay);
    *out = lay.pub;
    return LLSA_OK;
}

int llsa_workspace_layout(int B, int H, int N, int d, int block_size, int topk, int levels,
                          int dtype, llsa_ws_layout* out)
{
    return llsa_workspace_layout_lk(B, H, N, d, block_size, UniformK(topk, levels).ks, levels,
                                    dtype, out);
}

int llsa_zorder(const void* src, void* dst, long long outer, int side, int inner_bytes,
                int inverse, void* stream)
{
    if (!src || !dst) return LLSA_ERR_NULL;
    if (outer < 1 || side < 1 || side > (1 << 15) || !pow2(side) || inner_bytes < 4 ||
        inner_bytes % 4)
        return LLSA_ERR_SHAPE;
    return hip_rc(launch_zorder(src, dst, outer, side, inner_bytes, inverse,
                                (hipStream_t)stream));
}

int llsa_grid_order(const void* src, void* dst, long long outer, int frames, int height,
                    int width, int inner_bytes, int inverse, void* stream)
{
    if (!src || !dst) return LLSA_ERR_NULL;
    const int lim = 1 << 15;
    if (outer < 1 || frames < 1 || height < 1 || width < 1 || frames > lim || height > lim ||
        width > lim || (long long)frames * height * width > (1ll << 30) || inner_bytes < 4 ||
        inner_bytes % 4)
        return LLSA_ERR_SHAPE;
    return hip_rc(launch_grid_order(src, dst, outer, frames, height, width, inner_bytes, inverse,
                                    (hipStream_t)stream));
}

int llsa_forward_part(int part, const void* q, const void* k, const void* v, void* out,
                      float* lse, int B, int H, int N, int d, int block_size, int topk,
                      int levels, int dtype, unsigned flags, void* workspace, size_t ws_bytes,
                      void* stream)
{
    if (any_bad16(q, k, v, out) || bad_lse(lse)) return LLSA_ERR_NULL;
    Prep p;
    int rc = prepare(B, H, N, d, block_size, UniformK(topk, levels).ks, levels, dtype, flags,
                     workspace, ws_bytes, stream, &p);
    if (rc) return rc;
    return run_forward_part(part, q, k, v, out, lse, dtype, p);
}

int llsa_forward_lk(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int H, int N, int d, int block_size, const int* topk, int levels, int dtype,
                    unsigned flags, void* workspace, size_t ws_bytes, void* stream)
{
    if (any_bad16(q, k, v, out) || bad_lse(lse)) return LLSA_ERR_NULL;
    Prep p;
    int rc = prepare(B, H, N, d, block_size, topk, levels, dtype, flags, workspace, ws_bytes,
                     stream, &p);
    if (rc) return rc;
    return run_forward(q, k, v, out, lse, dtype, p);
}

int llsa_forward_grid(const void* q_raster, const void* k_raster, const void* v_raster,
                      void* q, void* k, void* v, void* out, float* lse, int B, int H,
                      int frames, int height, int width, int d, int block_size, int topk,
                      int levels, int dtype, unsigned flags, void* workspace,
                      size_t ws_bytes, void* stream)
{
    if (any_bad16(q_raster, k_raster, v_raster, q, k, v, out) || bad_lse(lse))
        return LLSA_ERR_NULL;
    const int lim = 1 << 15;
    if (frames < 1 || height < 1 || width < 1 || frames > lim || height > lim || width > lim ||
        (long long)frames * height * width > (1ll << 30))
        return LLSA_ERR_SHAPE;
    const int N = (int)((long long)frames * height * width);  // <= 2^30; validate caps it
    Prep p;
    int rc = prepare(B, H, N, d, block_size, UniformK(topk, levels).ks, levels, dtype, flags,
                     workspace, ws_bytes, stream, &p);
    if (rc) return rc;
    rc = hip_rc(launch_pool_gather(q_raster, k_raster, v_raster, q, k, v,
                                   make_grid_geo(frames, height, width), dtype, p.geo, p.ws, p.st));
    if (rc) return rc;
    rc = hip_rc(launch_select(p.geo, p.ws, false, p.st));
    if (rc) return rc;
    return run_forward_part(LLSA_PART_ATTN, q, k, v, out, lse, dtype, p);
}

int llsa_forward(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int H, int N, int d, int block_size, int topk, int levels, int dtype,
                 unsigned flags, void* workspace, size_t ws_bytes, void* stream)
{
    return llsa_forward_lk(q, k, v, out, lse, B, H, N, d, block_size,
                           UniformK(topk, levels).ks, levels, dtype, flags, workspace, ws_bytes,
                           stream);
}

int llsa_forward_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int H, int N, int d, int block_size, int topk, int levels,
                         int dtype, unsigned flags, void* stream)
{
    if (any_bad16(q, k, v, out) || bad_lse(lse)) return LLSA_ERR_NULL;
    const UniformK ks(topk, levels);
    int rc = validate(B, H, N, d, block_size, ks.ks, levels, dtype, flags);
    if (rc) return rc;
    Layout lay;
    make_layout(B * H, N, d, ks.ks, levels, &lay, true);
    if (lay.pub.total > (size_t)LLSA_NOALLOC_SCRATCH_BYTES) return LLSA_ERR_SCRATCH;
    void* base = nullptr;
    rc = noalloc_scratch(&base);
    if (rc) return rc;
    Prep p;
    rc = prepare(B, H, N, d, block_size, ks.ks, levels, dtype, flags, base,
                 (size_t)LLSA_NOALLOC_SCRATCH_BYTES, stream, &p, true);
    if (rc) return rc;
    // the pool launch zeroes the pick counters left by the previous call
    return run_forward(q, k, v, out, lse, dtype, p);
}

int llsa_backward_part(int part, const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                       int H, int N, int d, int block_size, int topk, int levels, int dtype,
                       unsigned flags, void* workspace, size_t ws_bytes, void* stream)
{
    if (any_bad16(q, k, v, out, dout, dq, dk, dv) || bad_lse(lse)) return LLSA_ERR_NULL;
    Prep p;
    int rc = prepare(B, H, N, d, block_size, UniformK(topk, levels).ks, levels, dtype, flags,
                     workspace, ws_bytes, stream, &p);
    if (rc) return rc;
    return run_backward_part(part, q, k, v, out, lse, dout, dq, dk, dv, dtype, p);
}

int llsa_backward_lk(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                     int H, int N, int d, int block_size, const int* topk, int levels,
                     int dtype, unsigned flags, void* workspace, size_t ws_bytes, void* stream)
{
    if (any_bad16(q, k, v, out, dout, dq, dk, dv) || bad_lse(lse)) return LLSA_ERR_NULL;
    Prep p;
    int rc = prepare(B, H, N, d, block_size, topk, levels, dtype, flags, workspace, ws_bytes,
                     stream, &p);
    if (rc) return rc;
    if (dtype == LLSA_BF16) {
        // dQ carries the first transpose launch's workgroups (one launch for
        // both); then the finer levels' transposes, if any
        rc = hip_rc(launch_attn_dq_transpose(q, k, v, out, lse, dout, dq, p.geo, p.ws, p.st));
        if (rc) return rc;
    } else {
        for (int part : {LLSA_PART_TRANSPOSE, LLSA_PART_DQ}) {
            rc = run_backward_part(part, q, k, v, out, lse, dout, dq, dk, dv, dtype, p);
            if (rc) return rc;
        }
    }
    for (int part : {LLSA_PART_ENRICH, LLSA_PART_DKDV}) {
        rc = run_backward_part(part, q, k, v, out, lse, dout, dq, dk, dv, dtype, p);
        if (rc) return rc;
    }
    return LLSA_OK;
}

int llsa_backward(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                  int H, int N, int d, int block_size, int topk, int levels, int dtype,
                  unsigned flags, void* workspace, size_t ws_bytes, void* stream)
{
    return llsa_backward_lk(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, block_size,
                            UniformK(topk, levels).ks, levels, dtype, flags, workspace,
                            ws_bytes, stream);
}

const char* llsa_strerror(int code)
{
    switch (code) {
    case LLSA_OK: return "ok";
    case LLSA_ERR_NULL: return "a required pointer is NULL or misaligned";
    case LLSA_ERR_SHAPE:
        return "bad shape: N a multiple of 16; B, H, levels >= 1; every top-k >= 1 and "
               "at most the candidates a row of its level may have (ceil(N/16^levels) at the "
               "coarsest level; below it 16 (parent top-k - 1) plus the children of the "
               "partial last parent); grid order: sides in [1, 2^15], at most 2^30 cells, "
               "inner_bytes a positive multiple of 4";
    case LLSA_ERR_UNSUPPORTED:
        return "unsupported: needs d=64 or 128, block_size=16, dtype f32/bf16, known flags, "
               "levels<=6, at most 4096 coarsest blocks, topk<=64, B*H*N<2^31, "
               "at most 2048 complement entries, no complement with causal";
    case LLSA_ERR_WORKSPACE: return "workspace missing or smaller than llsa_workspace_bytes()";
    case LLSA_ERR_HIP: return "HIP launch or runtime error";
    case LLSA_ERR_SCRATCH:
        return "llsa_forward_noalloc: this shape's forward state exceeds the static scratch "
               "of LLSA_NOALLOC_SCRATCH_BYTES (64 MiB); use llsa_forward with a workspace";
    default: return "unknown error code";
    }
}

}  // extern "C"
