/*
 * sva.h — block-sparse video self-attention on MI355X (gfx950).
 *
 * One attention call of a video diffusion transformer over T×Hh×W latent
 * tokens (plus optional extra audio/text tokens), in four calls:
 *
 *   sva_qk_norm_rope   QK-RMSNorm + 3D-RoPE on Q and K, fused in one kernel
 *   sva_reorder        raster tokens -> 3D-tile order (and back for O)
 *   sva_select_blocks  mean-pooled block scores, top-k key blocks per
 *                      query block and head
 *   sva_attention      online-softmax attention over the kept blocks only
 *
 * or in one: sva_forward runs the whole step with the fused variants of
 * these calls.
 *
 * Sources of the operations (web pages on the subject):
 *  - "MiniMax-H3 在 8×H200 上基准测试" (SGLang Diffusion benchmark),
 *    section "内核层": QK RMSNorm and 3D RoPE fused in one kernel, with the
 *    exact rounding path that rounds after the norm, before the rotation;
 *    section "SubBlock 稀疏注意力如何工作": a pooled score ranks the key
 *    blocks of each query block and head, the top ones are kept, their
 *    indices drive a block-sparse attention kernel, the full attention
 *    matrix is never built; sparsity is the fraction of key blocks dropped;
 *    the sparse path serves non-causal bf16 attention with head dim 128 and
 *    falls back to dense attention otherwise.
 *  - "Sol Video Inference Engine" blog, section 4.2.2: sparse attention
 *    cuts the quadratic cost of full spatiotemporal attention; Sparse
 *    VideoGen2 permutes tokens for the GPU layout.
 *
 * Conventions
 *  - All tensors are bf16 (uint16 storage), dense, 16-byte aligned, in
 *    device memory owned by the caller:
 *      raster      [B, N, H, d]    token n = (t·Hh + h)·W + w, then extras
 *      tile order  [B, H, Np, d]   Q, K and O after sva_reorder
 *      V tiles     [B, H, nB, block/32, 4, d, 8]   V after SVA_FORWARD_VT:
 *                                  each key block as groups of 32 keys, each
 *                                  group as four chunks of 8 keys, each chunk
 *                                  channel-major (d rows of 8 keys); chunk
 *                                  kc holds keys 16(kc/2) + 4(kc%2) +
 *                                  {0,1,2,3,8,9,10,11} of the group, in that
 *                                  order (the order the attention kernel's
 *                                  matrix instructions consume them in)
 *      K tiles     [B, H, nB, block/32, d/16, 64, 8]   K after SVA_FORWARD_KT:
 *                                  per 32-key group and 16-channel step s,
 *                                  64 entries of 8 channels; entry 32·hf + j
 *                                  holds key j of the group, channels
 *                                  16s + 8hf .. 16s + 8hf + 7
 *  - Np = n_video rounded up to a multiple of block, plus n_extra; nB =
 *    Np / block.  Padding rows of a tile-ordered tensor are zero.
 *  - Compute calls only enqueue work on `stream` (a hipStream_t; NULL is the
 *    default stream) and never synchronise.  Argument errors are detected on
 *    the host before anything is enqueued.  A plan is read-only after
 *    creation, so it may be used from several streams at once as long as
 *    each call gets its own output and workspace buffers.
 *  - Every call returns an SVA_* status; sva_last_error() gives a
 *    thread-local description of the last failure.
 */
#ifndef SVA_H
#define SVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define SVA_OK               0
#define SVA_ERR_INVALID_ARG -1  /* bad size, null/misaligned pointer, bad option */
#define SVA_ERR_UNSUPPORTED -2  /* head dim or block size the kernels do not
                                   serve (d, block not in {64, 128}); callers
                                   fall back to dense attention elsewhere */
#define SVA_ERR_WORKSPACE   -3  /* workspace smaller than required */
#define SVA_ERR_HIP         -4  /* HIP runtime error (allocation, launch) */

/* ---- plan flags ---- */
#define SVA_DENSE            1u /* keep every key block (same as sparsity 0):
                                   the dense warm-up steps of the pages */
#define SVA_KEEP_SAME_FRAME  2u /* always keep key blocks whose frame range
                                   meets the query block's frame range */
#define SVA_COMPENSATE       4u /* the step uses sva_attention_compensated:
                                   dropped key blocks enter the softmax as
                                   their mean key and value, weighted by size */

/* ---- block scorers (sva_plan_desc.scorer) ---- */
#define SVA_SCORER_MEAN      0  /* score = mean(Q' of qb) · mean(K' of kb)     */
#define SVA_SCORER_SUBBLOCK  1  /* "SubBlock 稀疏注意力如何工作": each block split
                                   into `subblocks` runs of consecutive tile-order
                                   tokens, pooled; score = log sum_a sum_b c_a c_b
                                   exp(qbar_a · kbar_b / sqrt(d)) over the runs'
                                   valid counts c (an estimate of the key block's
                                   unnormalised softmax mass for the query block) */

/* ---- sva_reorder directions ---- */
#define SVA_FORWARD     0  /* raster [B,N,H,d] -> tile order [B,H,Np,d]      */
#define SVA_INVERSE     1  /* tile order [B,H,Np,d] -> raster [B,N,H,d]      */
#define SVA_FORWARD_VT  2  /* raster [B,N,H,d] -> V tiles [B,H,nB,block/32,4,d,8] */
#define SVA_FORWARD_KT  3  /* raster [B,N,H,d] -> K tiles [B,H,nB,block/32,d/16,64,8] */
#define SVA_ROWS_TO_VT  4  /* tile order [B,H,Np,d] -> V tiles (as SVA_FORWARD_VT) */
#define SVA_ROWS_TO_KT  5  /* tile order [B,H,Np,d] -> K tiles (as SVA_FORWARD_KT) */

/* ---- output layouts of sva_attention_ex ---- */
#define SVA_LAYOUT_TILE    0   /* O in tile order [B, H, Np, d], padding rows zero */
#define SVA_LAYOUT_RASTER  1   /* O in raster order [B, N, H, d] (the inverse
                                  reorder fused into the attention)            */

typedef struct sva_plan_s* sva_plan;

/* Full description of a call.  Fill with sva_plan_desc_init() and change
 * what differs; zero-valued optional fields take the defaults below. */
typedef struct {
    int B, H;             /* batch, heads                                   */
    int T, Hh, W;         /* latent grid: frames, height, width             */
    int d;                /* head dim: 64 or 128                            */
    int block;            /* tokens per block: 64 or 128                    */
    double sparsity;      /* fraction of key blocks dropped, in [0, 1)      */
    unsigned flags;       /* SVA_DENSE | SVA_KEEP_SAME_FRAME                */
    int tile_t, tile_h, tile_w; /* 3D tile; 0,0,0 = 4×4×4 (block 64) or
                                   2×8×8 (block 128)                        */
    int n_extra;          /* extra tokens after the video tokens, a multiple
                             of block; their query rows and key columns are
                             always dense and they get no RoPE              */
    double rope_theta;    /* RoPE base; 0 = 10000                           */
    int rope_split[3];    /* channels for the t, h, w sections, each even;
                             sum <= d, channels past the sum are not rotated;
                             0,0,0 = 16/24/24 (d=64) or 44/42/42 (d=128)    */
    double eps;           /* RMSNorm epsilon; 0 = 1e-6                      */
    int scorer;           /* SVA_SCORER_MEAN (0) or SVA_SCORER_SUBBLOCK     */
    int subblocks;        /* SubBlock scorer: runs per block, 1, 2 or 4;
                             0 = 4 (the pages' 16-token sub-blocks of
                             64-token blocks); must be 0 or 1 for the mean
                             scorer                                          */
    int budget_multiple;  /* round the budget k up to a multiple of this
                             (the pages' SubBlock router uses 8); 0 = 1     */
} sva_plan_desc;

/* Sizes derived from a description. */
typedef struct {
    int64_t n_video;      /* T·Hh·W                                         */
    int64_t N;            /* n_video + n_extra (raster tokens)              */
    int64_t n_video_pad;  /* n_video rounded up to a multiple of block      */
    int64_t Np;           /* n_video_pad + n_extra (tile-ordered rows)      */
    int32_t nB;           /* Np / block                                     */
    int32_t nB_video;     /* n_video_pad / block                            */
    int32_t k;            /* key-block budget per row: ceil((1-sparsity)·nB)
                             rounded up to a multiple of budget_multiple,
                             clamped to [1, nB]; nB when dense              */
    int32_t max_row_len;  /* longest row of the block list                  */
    int64_t nnz_per_head; /* kept (query block, key block) pairs per (b, h) */
    int64_t nnz;          /* B·H·nnz_per_head: length of the col array      */
    size_t select_workspace_bytes; /* workspace sva_select_blocks needs     */
    int32_t dense;        /* 1 when every block is kept (no selection)      */
    int32_t tile[3];      /* resolved tile                                  */
    int32_t rope_split[3];/* resolved RoPE split                            */
    int32_t scorer;       /* resolved scorer                                */
    int32_t subblocks;    /* resolved runs per block (1 for the mean scorer) */
    int32_t budget_multiple; /* resolved budget multiple                    */
    int32_t n_mean_groups;/* ceil(nB / 32): groups of 32 block means in the
                             mean tiles of sva_block_means                  */
    size_t attention_workspace_bytes; /* workspace sva_attention_ws uses to
                             split long rows (0: no row is split)           */
} sva_plan_info;

/* ---- host-only calls (no device needed) ---- */

/* Fill `desc` with the given shape and defaults for everything else. */
int sva_plan_desc_init(sva_plan_desc* desc, int B, int H, int T, int Hh, int W,
                       int d, int block, double sparsity, unsigned flags);

/* Validate `desc` and compute its sizes into `info`. */
int sva_plan_query(const sva_plan_desc* desc, sva_plan_info* info);

/* Host copies of the plan's fixed tables, each optional (NULL skips it):
 *   perm     [N]       tile-order position of raster token n
 *   row_ptr  [nB + 1]  block-list row offsets, shared by every (b, h):
 *                      row qb of head (b, h) is col[(b·H + h)·nnz_per_head
 *                      + row_ptr[qb] .. + row_ptr[qb + 1]]
 *   forced   [nB·nB]   1 where key block kb is always kept for query block
 *                      qb (extra tokens, same frame); dense rows are all 1 */
int sva_plan_host_tables(const sva_plan_desc* desc, int32_t* perm,
                         int32_t* row_ptr, uint8_t* forced);

/* ---- plan lifetime (bound to the current HIP device) ---- */

/* Shape-only plan with default options (see sva_plan_desc_init). */
int sva_plan_create(sva_plan* out, int B, int H, int T, int Hh, int W, int d,
                    int block, double sparsity, unsigned dense_flag);
int sva_plan_create_ex(sva_plan* out, const sva_plan_desc* desc);
int sva_plan_get_info(sva_plan plan, sva_plan_info* info);
/* Frees the plan's device tables.  No work using the plan may be in flight. */
int sva_destroy(sva_plan plan);

/* ---- compute calls ---- */

/* QK-RMSNorm + 3D-RoPE (fused).  Per (token, head) row x of q and of k:
 *   y = bf16(x / sqrt(mean(x²) + eps) · w[h])      (norm, rounded first)
 *   out = bf16(rotate(y))                           (then RoPE, rounded)
 * where rotate turns channel pairs (2i, 2i+1) of the t, h and w sections by
 * coordinate · theta^(-2i/width); extra tokens are not rotated.
 * q, k, q_out, k_out: raster [B, N, H, d] bf16; wq, wk: [H, d] float32 or
 * NULL for ones.  In place (q_out == q, k_out == k) is allowed. */
int sva_qk_norm_rope(sva_plan plan, const void* q, const void* k,
                     const float* wq, const float* wk, void* q_out, void* k_out,
                     void* stream);

/* The same prologue written straight into the layouts the rest of the step
 * reads (the reorders of Q' and K' fused away): q_r = Q' in tile order
 * [B, H, Np, d], k_t = K' as K tiles (the layouts of SVA_FORWARD and
 * SVA_FORWARD_KT), padding rows zero.  Bit-identical to sva_qk_norm_rope
 * followed by those reorders.  The outputs must not overlap the inputs.
 * workspace (optional, device, workspace_bytes >= info.select_workspace_bytes):
 * when given for a sparse plan, the kernel also pools what it writes into
 * the block means that sva_select_blocks ranks ("lightweight pooling" of
 * the SubBlock section, fused into the producer), so the selection need
 * not read Q' and K' again: call sva_select_blocks with q_r = k_t = NULL
 * and the same workspace.  Ignored for a dense plan; NULL skips it. */
int sva_qk_norm_rope_tiled(sva_plan plan, const void* q, const void* k,
                           const float* wq, const float* wk, void* q_r, void* k_t,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Token permutation between raster and 3D-tile order (see direction
 * macros).  Forward writes zeros into the padding rows; the inverse drops
 * them.  SVA_ROWS_TO_KT and SVA_ROWS_TO_VT take K or V already in tile order
 * [B, H, Np, d] (as SVA_FORWARD writes it) and lay each block out as the
 * K or V tiles sva_select_blocks and sva_attention read, padding rows zero:
 * the output equals SVA_FORWARD_KT / SVA_FORWARD_VT of the raster tensor
 * the rows came from, so a caller holding k_r and v_r in tile order
 * converts them once and calls the rest of the step unchanged.  `in` and
 * `out` must not overlap. */
int sva_reorder(sva_plan plan, const void* in, void* out, int direction, void* stream);

/* Block selection.  q_r: tile order [B, H, Np, d] (SVA_FORWARD of Q');
 * k_t: K tiles (SVA_FORWARD_KT of K', the same buffer sva_attention reads).
 * q_r and k_t both NULL: the workspace already holds the block means,
 * written by sva_qk_norm_rope_tiled with this workspace (only the ranking
 * runs); one of them NULL is an argument error.
 * For every (b, h, query block qb): score(kb) by the plan's scorer (means
 * over valid tokens, float64); keep the forced blocks and then the
 * best-scored blocks (score descending, lower block index first on
 * equal scores) until the row holds row_ptr[qb+1] - row_ptr[qb] blocks.
 * Writes `col` [nnz] int32, each row in ascending block order.  `workspace`
 * (device, info.select_workspace_bytes) holds the block means.  Nothing to
 * do for a dense plan (col may be NULL). */
int sva_select_blocks(sva_plan plan, const void* q_r, const void* k_t,
                      void* workspace, size_t workspace_bytes, int32_t* col,
                      void* stream);

/* Block selection that allocates nothing, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The same selection as
 * sva_select_blocks with q_r and k_t given (pooling, then ranking), with
 * the block means kept in a fixed device array of the library instead of
 * a caller workspace: 128 MiB per GPU, held from the first plan created on
 * that GPU until the process ends.  A plan whose
 * info.select_workspace_bytes exceeds 128 MiB gets SVA_ERR_WORKSPACE before
 * anything is enqueued (the mean scorer fits up to 48 heads × 1024 blocks
 * at d = 128).  q_r, k_t and col as for sva_select_blocks (both inputs
 * required); the current device must be the plan's.  Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other threads) race and may return wrong lists; order them on one
 * stream.  Nothing to do for a dense plan. */
int sva_select_blocks_noalloc(sva_plan plan, const void* q_r, const void* k_t, int32_t* col,
                              void* stream);

/* Attention over the kept blocks.  For each valid query row p of block qb:
 * o_p = sum_j softmax_j(q_p·k_j / sqrt(d)) v_j over the valid keys j of the
 * blocks in row qb of `col` (any ascending list with the plan's row_ptr is
 * accepted; entries outside [0, nB) are skipped, and a row left with no
 * valid entry gets zero output; a dense plan ignores `col`, which may be
 * NULL).  q_r: [B, H, Np, d] (SVA_FORWARD of Q');
 * k_t: K tiles (SVA_FORWARD_KT of K'); v_t: V tiles (SVA_FORWARD_VT of V);
 * o_r: [B, H, Np, d], padding rows written as zero. */
int sva_attention(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                  const int32_t* col, void* o_r, void* stream);

/* sva_attention_ex with long rows split over several workgroups.  Rows
 * that keep every key block (the extra-token rows of a sparse plan) can be
 * many times longer than the video rows; walked by one workgroup each they
 * bound the step when there are few heads.  With a workspace of at least
 * info.attention_workspace_bytes (device memory, 16-byte aligned) every
 * row longer than 1.5 times the longest video row is cut into pieces of
 * at most that many list entries: each piece keeps its own running max m,
 * sum l and unnormalised output O (float32, in the workspace), and a merge
 * writes o = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i, M = max_i m_i
 * (the online-softmax merge of partial results; the rows it serves are
 * those of the audio tokens that the "内核层" section of the MiniMax-H3
 * page packs into one sequence with the video tokens).  The result equals
 * sva_attention_ex up to float rounding
 * order.  workspace NULL, or a plan with attention_workspace_bytes == 0:
 * exactly sva_attention_ex.  Other arguments as for sva_attention_ex;
 * compensated plans compensate the unsplit rows only (a split row keeps
 * every block). */
int sva_attention_ws(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                     const int32_t* col, const void* km_t, const void* vm_t, void* o,
                     int o_layout, void* workspace, size_t workspace_bytes, void* stream);

/* Block means for compensation.  From the K tiles and V tiles of a step,
 * the mean key and mean value of every key block over its valid tokens
 * (float32 sums, rounded to bf16), written as mean tiles in the layouts of
 * the K and V tiles with block kb as "key" kb % 32 of group kb / 32:
 *   km_t [B, H, n_mean_groups, d/16, 64, 8]    (K-tile layout)
 *   vm_t [B, H, n_mean_groups, 4, d, 8]        (V-tile layout)
 * Entries past nB are zero.  Caller-owned device buffers. */
int sva_block_means(sva_plan plan, const void* k_t, const void* v_t, void* km_t, void* vm_t,
                    void* stream);

/* Attention with compensation for the dropped blocks.  As sva_attention,
 * and every key block that row qb of `col` does not list enters the
 * softmax of each query of qb as one extra key: logit
 * q·kbar_B / sqrt(d) + ln|B| (|B| = the block's valid tokens) with value
 * vbar_B, from the mean tiles of sva_block_means.  The pages name a
 * light-weight compensation of the dropped blocks (Sol-Attn, "Sol Video
 * Inference Engine" README) and a first-order Taylor compensation (PISA,
 * "Sol Video Inference Engine" blog, 4.2.2); this is the leading term of
 * that expansion.  Dense rows have nothing to compensate. */
int sva_attention_compensated(sva_plan plan, const void* q_r, const void* k_t,
                              const void* v_t, const int32_t* col, const void* km_t,
                              const void* vm_t, void* o_r, void* stream);

/* General attention entry: km_t, vm_t both NULL (sva_attention) or both the
 * mean tiles of sva_block_means (sva_attention_compensated); o_layout
 * SVA_LAYOUT_TILE writes O like sva_attention, SVA_LAYOUT_RASTER writes
 * it in raster order [B, N, H, d], bit-identical to SVA_INVERSE of the
 * tile-order output. */
int sva_attention_ex(sva_plan plan, const void* q_r, const void* k_t, const void* v_t,
                     const int32_t* col, const void* km_t, const void* vm_t, void* o,
                     int o_layout, void* stream);

/* ---- the whole step ---- */

/* Device buffers of one sva_forward call: caller-owned device memory,
 * 16-byte aligned (col 4-byte), shapes as for the calls named there. */
typedef struct {
    const void* q;           /* raster [B, N, H, d] bf16 inputs                */
    const void* k;
    const void* v;
    const float* wq;         /* [H, d] float32 norm weights, or NULL for ones  */
    const float* wk;
    void* q_r;               /* written: Q' in tile order [B, H, Np, d]        */
    void* k_t;               /* written: K' as K tiles                         */
    void* v_t;               /* written: V as V tiles                          */
    void* select_ws;         /* sparse plans: info.select_workspace_bytes      */
    size_t select_ws_bytes;
    int32_t* col;            /* sparse plans, written: [nnz] kept block lists  */
    void* km_t;              /* compensated plans, written: mean tiles; else   */
    void* vm_t;              /*   NULL                                         */
    void* attn_ws;           /* optional: info.attention_workspace_bytes, or   */
    size_t attn_ws_bytes;    /*   NULL (no row split)                          */
    void* o;                 /* written: O in raster order [B, N, H, d]        */
} sva_step_buffers;

#define SVA_FORWARD_MARKS 6

/* The whole step in one call, on `stream`: sva_qk_norm_rope_tiled
 * (writing the block means for a sparse plan), sva_reorder(SVA_FORWARD_VT)
 * of v, sva_select_blocks from the means (sparse plans),
 * sva_block_means (compensated plans) and sva_attention_ws with O in
 * raster order; the results are those of these calls made in this order.
 * marks: NULL, or SVA_FORWARD_MARKS hipEvent_t created by the caller (NULL
 * entries skipped), recorded on `stream` at [0] the start and after [1] the
 * prologue, [2] the V reorder, [3] the selection, [4] the block means and
 * [5] the attention (an absent stage leaves two marks together), so one
 * call is timed stage by stage.  Argument errors as for the calls named,
 * all detected on the host before anything is enqueued.  The call only
 * launches kernels (and records the marks): it allocates, clears and
 * synchronises nothing, so with marks NULL it can be captured into a HIP
 * graph and replayed, the buffers staying bound to the captured pointers. */
int sva_forward(sva_plan plan, const sva_step_buffers* buffers, void* const* marks,
                void* stream);

/* ---- measurement ---- */

/* Plain device-to-device copy of `bytes` bytes (dst, src: device memory,
 * 16-byte aligned, not overlapping), enqueued on `stream`.  It is the
 * reference the HBM-bound kernels of the step are measured against: the
 * read + write rate a streaming kernel reaches on this part (16-byte
 * accesses, four per thread in flight, non-temporal hints), and a kernel
 * whose byte count is known, so profiler byte counters can be scaled by
 * it.  Not part of the attention step. */
int sva_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* ---- debug build ---- */

/* Built with -DSVA_DEBUG (libsva_debug.so: `python -m
 * block_sparse_attention_qk_amd.build --debug`), the kernels check the
 * indices they take from the plan's tables and from the block lists, and the
 * lists the selection writes.  A failed check sets its bit in the plan's
 * debug word (a 4-byte device word the plan owns, zero at creation) and the
 * kernel goes on: nothing traps.  Release builds carry no checks.  Bits: */
#define SVA_DEBUG_TOKEN 1u  /* a token index from the plan's permutation
                               tables outside its range */
#define SVA_DEBUG_LIST 2u   /* a block list row the selection wrote: an entry
                               outside [0, nB), or not exactly the row length */
#define SVA_DEBUG_ROW 4u    /* an attention row or work item outside the plan
                               (query block, row length, split piece, slot) */
#define SVA_DEBUG_SELF 8u   /* set by sva_debug_selftest */

/* Waits for the device (hipDeviceSynchronize), stores the plan's debug word
 * in *flags and clears it.  SVA_ERR_UNSUPPORTED in a release build (then
 * *flags is 0). */
int sva_debug_flags(sva_plan plan, unsigned* flags);

/* Enqueues on `stream` one kernel whose check fails on purpose, so that the
 * next sva_debug_flags reports SVA_DEBUG_SELF: a test of the reporting path
 * itself.  SVA_ERR_UNSUPPORTED in a release build. */
int sva_debug_selftest(sva_plan plan, void* stream);

/* ---- errors ---- */
const char* sva_status_string(int status);
const char* sva_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SVA_H */
