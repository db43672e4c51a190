/*
 * llsa.h -- C ABI of libllsa.so, the MI355X (gfx950) implementation of the
 * hot path of Log-linear Sparse Attention (LLSA).
 *
 * The method (pages: the LLSA GitHub README, "usage" and "reordering"
 * sections; the LLSA skill summary, "Core Technique" 1-3; the arXiv 2512.16615
 * abstract):
 *   - tokens of a 2-D grid are put in Z-order (quadtree order) so that every
 *     run of 16^l consecutive tokens is a square tile;
 *   - queries and keys are block-mean-pooled into a pyramid (block_size 16);
 *   - Top-K key blocks are chosen per query block: densely at the coarsest
 *     level, and at every finer level only among the children of the blocks
 *     chosen one level up;
 *   - attention (non-causal; causal with LLSA_CAUSAL) runs over the tokens of
 *     the chosen level-1 blocks,
 *     enriched with the pooled key/value tokens of the blocks chosen at every
 *     level;
 *   - the backward pass turns the query->key block lists into key->query
 *     lists (a sparse index transpose) instead of building a dense mask.
 *
 * Token counts (README usage: the power-of-two limit is to be lifted).  N
 *   is any multiple of 16.  Level l has n_l = ceil(N / 16^l) blocks; when 16^l
 *   does not divide N the last one is partial, as if the sequence were padded
 *   to a multiple of 16^levels with tokens that are never attended: its pooled
 *   token is the mean of the tokens it covers (and passes 1/count of its
 *   gradient to each), and a level's candidates are the blocks that exist.  A
 *   row of the coarsest level chooses among n_L blocks; below it among the
 *   existing children of its parent's picks -- at worst 16 (topk_{l+1} - 1)
 *   full parents and the partial last one -- and top-k may not exceed that.
 *
 * Conventions shared by all entry points
 *   Tensors q, k, v, out, dout, dq, dk, dv: contiguous [B][H][N][d] in the
 *   element type `dtype` (LLSA_F32 or LLSA_BF16), tokens already in Z-order
 *   (see llsa_zorder).  lse: contiguous [B][H][N] float32, natural log of the
 *   softmax normaliser of each query row.
 *   Pointers to tensors and to the workspace are DEVICE pointers owned by the
 *   caller; the library never allocates, frees or keeps them.
 *   stream: a hipStream_t (NULL = the default stream).  Calls only enqueue
 *   work on that stream and return; nothing synchronises the host.
 *   Apart from llsa_forward_noalloc's static scratch (see there), the library
 *   holds no mutable global state: concurrent calls with distinct workspaces
 *   are safe.
 *   A workspace is trusted to hold what the forward of the same shape, dtype,
 *   top-k and flags left there: with other contents the results are wrong,
 *   but every index read from it is clamped to its range before it forms an
 *   address, so no access leaves the buffers the call was given.
 *   All argument validation happens before any HIP call, so every error code
 *   except LLSA_ERR_HIP can be observed without a GPU.
 */
#ifndef LLSA_H
#define LLSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define LLSA_F32 0
#define LLSA_BF16 1

/* flags: which pooled tokens enrich the key/value set (skill summary, "Core
 * Technique" 2, leaves the levels and the weighting open).  Default (0): the
 * pooled keys/values of the blocks chosen at every level, plain logits. */
#define LLSA_NO_ENRICH 1u     /* attend to the selected fine blocks only */
#define LLSA_ENRICH_COARSE 2u /* pooled tokens of levels 2..levels only */
#define LLSA_SIZE_BIAS 4u     /* a level-l pooled token, the mean of 16^l tokens,
                                 counts as 16^l copies (logit + ln 16^l) */
#define LLSA_ENRICH_COMPLEMENT 8u /* the pooled tokens of the candidates each level did
                                     NOT pick (every coarsest block not picked; below
                                     it the parent's picks' children not picked):
                                     with the fine tokens they cover every key token
                                     once.  At most 2048 such entries per query block
                                     (sum over the enriching levels of the candidate
                                     counts), else LLSA_ERR_UNSUPPORTED */
#define LLSA_CAUSAL 16u       /* causal attention (the README's usage note names the
                                 non-causal form only; this is the reading taken):
                                 token t attends keys u <= t.  At every level a
                                 query block keeps its own block and its best
                                 topk - 1 earlier candidates (all of them when
                                 fewer), the valid picks first, ascending, then -1
                                 in the slots left; the query's own fine block is
                                 masked to keys u <= t, and the pooled token of an
                                 ancestor's own block (its mean holds later tokens)
                                 does not enrich.  topk is limited as without
                                 the flag.  Not with LLSA_ENRICH_COMPLEMENT
                                 (LLSA_ERR_UNSUPPORTED) */
#define LLSA_KNOWN_FLAGS 31u

/* error codes */
#define LLSA_OK 0
#define LLSA_ERR_NULL (-1)        /* a required pointer is NULL, or a tensor
                                     pointer (q, k, v, out, dout, dq, dk, dv,
                                     the raster inputs) not 16-byte aligned,
                                     or lse not 4-byte aligned */
#define LLSA_ERR_SHAPE (-2)       /* levels < 1, N not a multiple of 16,
                                     a top-k < 1 or above the candidates a row
                                     of its level may have (see below),
                                     B or H < 1 (N and topk need not be
                                     powers of two, nor N a multiple of
                                     16^levels) */
#define LLSA_ERR_UNSUPPORTED (-3) /* d not 64 or 128, block_size != 16, unknown dtype
                                     or flags, levels > LLSA_MAX_LEVELS,
                                     coarsest block count > 4096, topk > 64,
                                     N > 2^23, or B*H*N >= 2^31 */
#define LLSA_ERR_WORKSPACE (-4)   /* workspace NULL, not 16-byte aligned, or
                                     smaller than llsa_workspace_bytes() */
#define LLSA_ERR_HIP (-5)         /* a HIP launch or runtime call failed */
#define LLSA_ERR_SCRATCH (-6)     /* llsa_forward_noalloc: the shape needs more
                                     than LLSA_NOALLOC_SCRATCH_BYTES */

#define LLSA_MAX_LEVELS 6

/* Byte offsets of the parts of the workspace (a test and profiling hook).
 * Level arrays are indexed by l - 1 for level l = 1..levels.
 *   qbar/kbar/vbar[l-1] : float32 [B*H][N/16^l][d]   block means (pyramid)
 *   idx[l-1]            : int32   [B*H][N/16^l][topk] chosen blocks of each
 *                         (topk: that level's count with the _lk calls)
 *                         level-l query block, ascending (LLSA_CAUSAL: -1 in
 *                         the unused slots after the picks)
 *   rowptr[l-1]         : int32   [B*H][N/16^l + 1]  key->query lists (CSR,
 *   col[l-1]            : int32   [B*H][N/16^l*topk]  offsets per head from 0,
 *                         each list ascending); written by llsa_backward
 *   delta               : float32 [B*H][N]  rowsum(dout * out), backward
 *   total               : bytes needed (== llsa_workspace_bytes) */
typedef struct {
    size_t qbar[LLSA_MAX_LEVELS];
    size_t kbar[LLSA_MAX_LEVELS];
    size_t vbar[LLSA_MAX_LEVELS];
    size_t idx[LLSA_MAX_LEVELS];
    size_t rowptr[LLSA_MAX_LEVELS];
    size_t col[LLSA_MAX_LEVELS];
    size_t delta;
    size_t total;
} llsa_ws_layout;

/* Bytes of device workspace llsa_forward / llsa_backward need for this shape
 * (O(B*H*N*d), never O(N^2): no dense mask).  Returns 0 for arguments that
 * llsa_forward would reject. */
size_t llsa_workspace_bytes(int B, int H, int N, int d, int block_size, int topk,
                            int levels, int dtype);

/* Fills *out with the workspace layout of this shape.  Returns LLSA_OK or the
 * validation error llsa_forward would return (out untouched then). */
int llsa_workspace_layout(int B, int H, int N, int d, int block_size, int topk,
                          int levels, int dtype, llsa_ws_layout* out);

/* Z-order (quadtree) token permutation (README, "reordering non-sequential
 * data": quadrants top-left, top-right, bottom-left, bottom-right at every
 * scale; Morton code with the row bit above the column bit).
 * src, dst: device buffers [outer][side*side][inner_bytes], must not overlap.
 * inverse == 0: raster -> Z-order, dst[o][morton(y,x)] = src[o][y*side+x];
 * inverse != 0: Z-order -> raster.
 * side must be a power of two in [1, 2^15]; inner_bytes a positive multiple
 * of 4.  Errors: LLSA_ERR_NULL, LLSA_ERR_SHAPE, LLSA_ERR_HIP. */
int llsa_zorder(const void* src, void* dst, long long outer, int side, int inner_bytes,
                int inverse, void* stream);

/* Grid order: the quadtree permutation extended to images whose sides are not
 * equal powers of two and, as an octree, to video (README: images or videos
 * are reordered so that nearby cells share blocks).  The grid of `frames`
 * frames of height x width cells (frames == 1: an image) is cut into tiles of
 * S x S cells (S x S x S when frames > 1), S the largest power of two that
 * divides every side; tiles are taken in raster order (frame, row, column)
 * and the cells of a tile in Morton order with, at every scale, the frame bit
 * above the row bit above the column bit.  A square power-of-two image gives
 * llsa_zorder's order.  With 4^l dividing the tile side, every aligned run of
 * 16^l tokens of an image is a 4^l x 4^l patch.
 * src, dst: device buffers [outer][frames*height*width][inner_bytes], not
 * overlapping; inverse == 0: raster -> grid order, else the inverse.
 * Each side in [1, 2^15], frames*height*width <= 2^30, inner_bytes a positive
 * multiple of 4.  Errors: LLSA_ERR_NULL, LLSA_ERR_SHAPE, LLSA_ERR_HIP. */
int llsa_grid_order(const void* src, void* dst, long long outer, int frames, int height,
                    int width, int inner_bytes, int inverse, void* stream);

/* LLSA forward: pyramid, hierarchical Top-K (scores s*<qbar, kbar> in fp32,
 * s = 1/sqrt(d), ties to the lower block index) and sparse attention with
 * enrichment (unless LLSA_NO_ENRICH) writing out [B][H][N][d] and lse.
 * The pyramid and the index lists are left in the workspace for
 * llsa_backward, which must get the same workspace, shape, dtype and flags.
 * levels = 1 corresponds to the README's llsa_l1, levels = 2 to llsa_l2. */
int llsa_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int H, int N, int d, int block_size, int topk, int levels,
                 int dtype, unsigned flags, void* workspace, size_t ws_bytes,
                 void* stream);

/* llsa_forward on raster-order inputs, the grid order folded into the
 * pooling pass (README, reordering of non-sequential data, then usage):
 * q_raster, k_raster, v_raster are [B][H][frames*height*width][d] in raster
 * order (frame, row, column).  The call writes their grid-ordered copies to
 * q, k, v -- the bytes llsa_grid_order would write, and what llsa_backward
 * takes -- while it pools them, so each input is read once, then selects and
 * attends exactly as llsa_forward on q, k, v (out, lse in grid order; the
 * same results bit for bit).  N = frames*height*width.  The raster buffers
 * must not overlap q, k, v.  Grid sides as for llsa_grid_order, and the
 * shape, top-k, flags and workspace as for llsa_forward.  Errors: those of
 * llsa_grid_order and llsa_forward. */
int llsa_forward_grid(const void* q_raster, const void* k_raster, const void* v_raster,
                      void* q, void* k, void* v, void* out, float* lse, int B, int H,
                      int frames, int height, int width, int d, int block_size, int topk,
                      int levels, int dtype, unsigned flags, void* workspace,
                      size_t ws_bytes, void* stream);

/* LLSA backward (skill summary, "Core Technique" 3): given dout, writes dq,
 * dk, dv ([B][H][N][d], dtype).  Reuses the forward's pyramid and index lists
 * from the workspace (no re-selection; selection passes no gradient), builds
 * the key->query lists by a counting sort, then computes dq query-major and
 * dk, dv key-major.  A pooled token passes 1/16^l of its gradient to each of
 * the 16^l tokens it averages.  Deterministic: no floating-point atomics. */
int llsa_backward(const void* q, const void* k, const void* v, const void* out,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  int B, int H, int N, int d, int block_size, int topk, int levels,
                  int dtype, unsigned flags, void* workspace, size_t ws_bytes,
                  void* stream);

/* A top-k per level (the README's usage takes one top-k for every level; the
 * hierarchical selection of the skill summary, "Core Technique" 1, works the
 * same with a different count at each level).  topk: HOST array of `levels`
 * ints, topk[l-1] the picks of every level-l row, level 1 (the fine blocks)
 * first; read during the call only.  Level l < levels chooses among the
 * (up to) 16*topk[l] children of its parent's picks, so 1 <= topk[l-1] <=
 * 16*(topk[l] - 1) + the children of the level's partial last parent (16 when
 * 16^(l+1) divides N); the coarsest level among ceil(N/16^levels) blocks.  Every other
 * argument, the layout and the errors are those of the uniform calls (a NULL
 * topk gives LLSA_ERR_NULL); with equal values the results are identical to
 * them.  The workspace must be sized by llsa_workspace_bytes_lk with the same
 * array, and the backward given the forward's array. */
size_t llsa_workspace_bytes_lk(int B, int H, int N, int d, int block_size, const int* topk,
                               int levels, int dtype);
int llsa_workspace_layout_lk(int B, int H, int N, int d, int block_size, const int* topk,
                             int levels, int dtype, llsa_ws_layout* out);
int llsa_forward_lk(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int H, int N, int d, int block_size, const int* topk, int levels, int dtype,
                    unsigned flags, void* workspace, size_t ws_bytes, void* stream);
int llsa_backward_lk(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                     int H, int N, int d, int block_size, const int* topk, int levels,
                     int dtype, unsigned flags, void* workspace, size_t ws_bytes, void* stream);

/* Stages of llsa_forward / llsa_backward, for per-kernel timing and tests.
 * llsa_forward gives the results of parts POOL, SELECT, ATTN in that order;
 * llsa_backward those of parts TRANSPOSE, DQ, ENRICH, DKDV in that order
 * (ENRICH: gradients of the pooled tokens, needed by DKDV).  The full calls
 * may merge launches (the bf16 backward runs TRANSPOSE's first levels inside
 * DQ's launch; the forward's pool zeroes SELECT's counters).  Each part reads what the parts before it
 * left in the workspace (SELECT also records how often each key block was
 * chosen, which TRANSPOSE uses); any part may be repeated.  Same arguments
 * and errors as the full calls; an unknown part number gives
 * LLSA_ERR_UNSUPPORTED. */
#define LLSA_PART_POOL 0
#define LLSA_PART_SELECT 1
#define LLSA_PART_ATTN 2
#define LLSA_PART_TRANSPOSE 3
#define LLSA_PART_DQ 4
#define LLSA_PART_DKDV 5
#define LLSA_PART_ENRICH 6
int llsa_forward_part(int part, const void* q, const void* k, const void* v, void* out,
                      float* lse, int B, int H, int N, int d, int block_size, int topk,
                      int levels, int dtype, unsigned flags, void* workspace,
                      size_t ws_bytes, void* stream);
int llsa_backward_part(int part, const void* q, const void* k, const void* v,
                       const void* out, const float* lse, const void* dout, void* dq,
                       void* dk, void* dv, int B, int H, int N, int d, int block_size,
                       int topk, int levels, int dtype, unsigned flags, void* workspace,
                       size_t ws_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and errors are llsa_forward's (outputs
 * identical bit for bit), without the workspace: the pyramid, index lists and
 * pick counters live in a static scratch array of LLSA_NOALLOC_SCRATCH_BYTES
 * in each GPU's memory, reserved when the library is loaded on that GPU and
 * held until the process ends.  The call itself allocates nothing.
 *   - Shapes whose forward state exceeds the array are refused with
 *     LLSA_ERR_SCRATCH before any launch (at d = 64: up to about 2^17 tokens
 *     times 6 heads at 2 levels, e.g. 256x256 with 6 heads, fits).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents (each call rewrites what it reads).  Calls that overlap
 *     in time on one GPU -- other streams, other host threads, other
 *     processes' streams do not share it -- race and give wrong results;
 *     calls ordered on one stream are safe.
 *   - There is no matching backward: the next call overwrites the index
 *     lists.  Training keeps using llsa_forward / llsa_backward. */
#define LLSA_NOALLOC_SCRATCH_BYTES (64u << 20)
int llsa_forward_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int H, int N, int d, int block_size, int topk, int levels,
                         int dtype, unsigned flags, void* stream);

/* Static description of an error code (never NULL). */
const char* llsa_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
