/*
 * liblcsa -- locality-constrained sparse attention (LCSA) for AMD Instinct
 * MI355X (gfx950): block selection and block-sparse attention over a latent
 * video token grid.
 *
 * The method: every query block keeps the k key blocks whose mean-pooled key
 * scores highest against its mean-pooled query, among the key blocks that lie
 * in a spatial window around it (any KV frame), and then attends with softmax
 * over the tokens of those blocks only.  Attention limited to spatially local
 * patches is LCSA as described in the agentlens FlashVSR summary ("How it
 * works", item 2); pooling, mask selection and the CSR form of the mask are the
 * attention glue named on the FlashVSR Hopper PR page ("What Was Actually
 * Slow", "Rebuild sparse attention for Hopper"); the controls topk_ratio,
 * local_range and kv_ratio come from the FlashVSR Inference skill page
 * ("Non-Negotiable Streaming Contract").
 *
 * Conventions shared by every entry point:
 *  - Tokens are in raster order (t, y, x) -> (t * grid_h + y) * grid_w + x,
 *    t counting latent frames.  Q covers the q_frames newest frames of the KV
 *    window; K and V cover all kv_frames frames of the window, oldest first.
 *  - Q, K, V, O are bf16 with logical shape [batch, tokens, heads, head_dim];
 *    head_dim is contiguous, other dims follow caller strides (elements).
 *  - Blocks are 1 frame x block_h x block_w tokens; block index
 *    kb = t * blocks_per_frame + by * (grid_w / block_w) + bx.
 *  - The CSR block mask has one row per (b, h, query block):
 *    row r = (b * heads + h) * nqb + qb; row_ptr has rows + 1 int32 entries;
 *    col_idx holds key-block indices, strictly ascending inside a row.
 *  - The library allocates no device memory.  The caller owns every buffer
 *    (inputs, outputs, CSR, workspace) and the stream.
 *  - All validation happens on the host before anything is enqueued; on an
 *    error nothing is enqueued and the status says why (lcsa_last_error() has
 *    the detail).  There is no fallback path of any kind.  Launches are
 *    asynchronous: device faults surface at the caller's next synchronisation.
 *  - No C++ exception crosses this interface.
 */
#ifndef LCSA_H_
#define LCSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCSA_ABI_VERSION 7

typedef int32_t lcsa_status;
#define LCSA_OK 0
#define LCSA_ERR_NULL 1       /* a required pointer is NULL */
#define LCSA_ERR_INVALID 2    /* a descriptor value is out of range */
#define LCSA_ERR_SHAPE 3      /* grid not tileable / sizes beyond limits /
                                 tensor extents differ from the plan's */
#define LCSA_ERR_ALIGN 4      /* data or strides not 16-byte aligned */
#define LCSA_ERR_WORKSPACE 5  /* workspace missing or too small */
#define LCSA_ERR_DEVICE 6     /* no current HIP device, or it is not gfx950 */
#define LCSA_ERR_LAUNCH 7     /* the HIP runtime rejected a launch */
#define LCSA_ERR_INTERNAL 8   /* allocation failure or unexpected state */

#define LCSA_DTYPE_BF16 1

/* Most KV-window frames a plan may have. */
#define LCSA_MAX_KV_FRAMES 64

/* Shape and control of one LCSA layer call.
 *  batch, heads       > 0.
 *  head_dim           must be 128 (the DiT's head size; NxDI FlashVSR
 *                     contrib page, "Model Information").
 *  grid_h, grid_w     tokens per latent frame (output pixels / 16).
 *  q_frames           latent frames of the current chunk (queries), > 0.
 *  cached_frames      earlier latent frames held in the KV cache, >= 0.
 *  kv_ratio           KV window length bound: kv_frames = min(cached_frames +
 *                     q_frames, ceil(kv_ratio * q_frames)); <= 0 means no
 *                     bound; a value in (0, 1) is invalid.
 *  block_t/h/w        block shape in tokens; all zero = automatic (1x8x16 if
 *                     it tiles the grid, else 1x16x8); block_t must be 0 or 1
 *                     and block_h * block_w must be 64 or 128.
 *  local_range        odd window width in blocks (>= 1); the window is every
 *                     KV frame and block rows/columns within local_range / 2.
 *  topk_ratio         budget k = round-half-up(topk_ratio * blocks per frame)
 *                     (values within 1e-9 of an integer snap to it), >= 1.
 *  topk               > 0 overrides topk_ratio with an explicit k.
 *  scale              softmax scale; 0 means 1 / sqrt(head_dim). */
typedef struct lcsa_desc {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t grid_h;
  int32_t grid_w;
  int32_t q_frames;
  int32_t cached_frames;
  int32_t block_t;
  int32_t block_h;
  int32_t block_w;
  int32_t local_range;
  int32_t topk;
  double topk_ratio;
  float kv_ratio;
  float scale;
} lcsa_desc;

/* A device tensor view of logical shape [batch, tokens, heads, head_dim].
 * data must be 16-byte aligned and stride_b/stride_s/stride_h (in elements)
 * multiples of 8, so that every (token, head) row is a 256-byte aligned-16
 * contiguous vector.  dtype must be LCSA_DTYPE_BF16.  The extents state the
 * view's logical shape; every call checks them against the plan (the plan's
 * batch and heads, head_dim 128, and the call's token count: q_tokens for
 * queries and outputs, kv_tokens for a contiguous K/V window, slots *
 * grid_h * grid_w for a frame ring) and returns LCSA_ERR_SHAPE on a
 * mismatch.  The library cannot see the allocation behind data: the caller
 * guarantees that every element the extents and strides address exists. */
typedef struct lcsa_tensor {
  void* data;
  int32_t dtype;
  int32_t reserved;
  int64_t stride_b;
  int64_t stride_s;
  int64_t stride_h;
  int64_t batch;
  int64_t tokens;
  int64_t heads;
  int64_t head_dim;
} lcsa_tensor;

/* Everything the plan derived from a descriptor. */
typedef struct lcsa_plan_info {
  int32_t kv_frames;
  int32_t blocks_per_frame;
  int32_t nbh;                 /* block rows per frame */
  int32_t nbw;                 /* block columns per frame */
  int32_t nqb;                 /* query blocks = q_frames * blocks_per_frame */
  int32_t nkb;                 /* key blocks = kv_frames * blocks_per_frame */
  int32_t k;                   /* budget before clamping to a row's window */
  int32_t block_h;
  int32_t block_w;
  int32_t block_tokens;
  int32_t half_window;         /* local_range / 2 */
  int32_t max_row_nnz;         /* largest min(k, |window|) over rows */
  int32_t min_window;          /* smallest window size over query blocks */
  int32_t max_window;          /* largest window size over query blocks */
  int64_t rows;                /* batch * heads * nqb */
  int64_t nnz;                 /* total selected blocks (row_ptr[rows]) */
  int64_t q_tokens;
  int64_t kv_tokens;
  uint64_t select_workspace_bytes;
  uint64_t attend_workspace_bytes; /* enough for any gfx950 device */
  uint64_t kcache_slot_bytes;  /* pooled-K cache bytes per ring slot */
  double scale;                /* softmax scale actually used */
  double useful_flops;         /* 4 * head_dim * block_tokens^2 * nnz */
} lcsa_plan_info;

typedef struct lcsa_plan_s* lcsa_plan_t;

/* Validate a descriptor and precompute geometry, budget, window sizes and the
 * CSR row pointer.  The controls are those of the streaming pipeline: the
 * kept-block budget from topk_ratio, the spatial window local_range and the
 * KV window length from kv_ratio (FlashVSR Inference skill page,
 * "Non-Negotiable Streaming Contract"), over chunks of latent frames (a
 * 6-frame first chunk and 2-frame stream chunks on the NxDI FlashVSR contrib
 * page, "Description").  Host only: needs no GPU.  On success *out owns a new
 * plan (release with lcsa_plan_destroy); it is immutable and may be shared
 * across threads and streams.  Errors: NULL, INVALID, SHAPE, INTERNAL. */
lcsa_status lcsa_plan_create(const lcsa_desc* desc, lcsa_plan_t* out);

/* Release a plan; NULL is a no-op. */
void lcsa_plan_destroy(lcsa_plan_t plan);

/* Copy the plan's derived values into *info.  Errors: NULL. */
lcsa_status lcsa_plan_get_info(lcsa_plan_t plan, lcsa_plan_info* info);

/* Copy the plan's CSR row pointer (rows + 1 int32 values, row r holds
 * min(k, |window(qb)|) blocks) into host memory.  capacity is the number of
 * int32 the caller provided.  Errors: NULL, WORKSPACE (capacity too small). */
lcsa_status lcsa_plan_row_ptr(lcsa_plan_t plan, int32_t* host_out, int64_t capacity);

/* Copy the window (eligible key blocks, ascending) of query block qb into
 * host memory; *count receives its size.  Errors: NULL, INVALID (qb out of
 * range), WORKSPACE (capacity smaller than the window). */
lcsa_status lcsa_plan_window(lcsa_plan_t plan, int32_t qb, int32_t* host_out,
                             int32_t capacity, int32_t* count);

/* Block selection: mean-pool K per key block and Q per query block
 * (float64 sums of the bf16 values), score each query block against every
 * key block of its window (float64 dot products), keep the k best
 * (descending score, ties to the lower block index) and emit them ascending
 * as the CSR block mask.  Pooling and mask selection are the attention glue
 * and the mask is built as CSR on the FlashVSR Hopper PR page ("What Was
 * Actually Slow"; "Rebuild sparse attention for Hopper"); candidates are the
 * key blocks of a spatial window around the query block (agentlens FlashVSR
 * summary, "How it works", item 2).
 *  q, k            device views (shape [batch, q_tokens | kv_tokens, heads,
 *                  128]), read only.
 *  d_row_ptr       device int32[rows + 1], written (equal to the plan's).
 *  d_col_idx       device int32[nnz], written.
 *  d_scores        NULL, or device double[batch * heads * nqb * nkb] that
 *                  receives every pooled score (-inf outside the window).
 *  d_workspace     device buffer of at least select_workspace_bytes bytes,
 *                  256-byte aligned; its contents are scratch.
 *  stream          hipStream_t to enqueue on (NULL = default stream).
 * Errors: NULL, ALIGN, SHAPE, WORKSPACE, DEVICE, LAUNCH. */
lcsa_status lcsa_select(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                        int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                        void* d_workspace, size_t workspace_bytes, void* stream);

/* Block selection that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments
 * (less the workspace) and same result as lcsa_select; the pooled vectors go
 * to a scratch array inside the library instead, of
 * LCSA_SELECT_NOALLOC_MAX_BYTES bytes on each device the library runs on,
 * held until the process ends.  The call itself allocates nothing.
 *  - A plan whose select_workspace_bytes exceeds
 *    LCSA_SELECT_NOALLOC_MAX_BYTES is rejected with LCSA_ERR_WORKSPACE
 *    before anything is enqueued (48 MiB holds the 184320-token 4K first
 *    chunk at 12 heads, 33.75 MiB).
 *  - All calls on one device share that device's one array: calls that
 *    overlap in time on one device (other streams, other host threads)
 *    race on it, and the caller must serialise them.  Each call writes every
 *    entry it later reads, so nothing carries over from an earlier call.
 * Errors: as lcsa_select (WORKSPACE only for the size limit). */
#define LCSA_SELECT_NOALLOC_MAX_BYTES (48ull << 20)
lcsa_status lcsa_select_noalloc(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                                int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                                void* stream);

/* Block-sparse attention forward: for each CSR row (b, h, query block) and
 * every token of every key block in the row, z = scale * q.k; online softmax
 * over those tokens; O = sum softmax(z) v, rounded to bf16 (nearest even);
 * LSE = max z + ln(sum exp(z - max z)) in float32.  The attention step of
 * LCSA: attention limited to the selected local blocks (agentlens FlashVSR
 * summary, "How it works", item 2) run as a block-sparse kernel over a CSR
 * block list (FlashVSR Hopper PR page, "Rebuild sparse attention for
 * Hopper").
 *  q, k, v, o      device views; o is written, the others are read.
 *  d_row_ptr       device int32[rows + 1]; d_col_idx device int32[nnz].
 *                  Any CSR is accepted: row bounds are clamped to [0, nnz]
 *                  and block indices outside [0, nkb) are skipped in the
 *                  kernel, so malformed content cannot read out of bounds.
 *                  A row with no valid block yields O = 0 and LSE = -inf.
 *  nnz             number of int32 in d_col_idx.
 *  d_lse           NULL, or device float[batch * heads * q_tokens].
 *  d_workspace     NULL, or a device buffer of workspace_bytes (256-byte
 *                  aligned, at least attend_workspace_bytes) for partial
 *                  results.  With it, the rows that would run in a last,
 *                  partly filled round of workgroups are split into pieces
 *                  over their block lists and merged by a second kernel;
 *                  without it, every row is one workgroup.  Results agree
 *                  to rounding; the contents are scratch.
 * Errors: NULL, ALIGN, INVALID (nnz < 0), SHAPE, WORKSPACE, DEVICE, LAUNCH. */
lcsa_status lcsa_attend(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                        const lcsa_tensor* v, const int32_t* d_row_ptr,
                        const int32_t* d_col_idx, int64_t nnz, const lcsa_tensor* o,
                        float* d_lse, void* d_workspace, size_t workspace_bytes,
                        void* stream);

/* Streaming KV storage.  In the streaming contract every chunk's queries
 * attend to a KV window of the newest kv_frames latent frames (FlashVSR
 * Inference skill page, "Non-Negotiable Streaming Contract": kv_ratio), and
 * KV concatenation and pooling of that window are part of the attention glue
 * (FlashVSR Hopper PR page, "What Was Actually Slow").  A frame ring avoids
 * both copies: K and V live frame by frame in `slots` ring slots of two
 * caller buffers (logical shape [batch, slots * grid_h * grid_w, heads,
 * 128], lcsa_tensor strides as usual), each chunk writes only its new
 * frames, and frame_slot[t] names the slot of window frame t (oldest first,
 * t < kv_frames).  Slot indices must lie in [0, slots). */
typedef struct lcsa_kv_ring {
  int32_t slots;
  int32_t frame_slot[LCSA_MAX_KV_FRAMES];
} lcsa_kv_ring;

/* Block selection over a frame ring with an incremental pooled-K cache.
 * Same result as lcsa_select on the window's K laid out contiguously.
 *  k_ring          the K ring (see lcsa_kv_ring), read only.
 *  new_frames      0 .. kv_frames: the pooled K of the new_frames newest
 *                  window frames is computed and stored in their slots'
 *                  cache entries; the entries of the older window frames
 *                  are used as they are, so they must hold the pooled K of
 *                  the frames now in those slots (written by an earlier
 *                  call with the same batch, heads and grid).
 *  d_kcache        device double[slots * kcache_slot_bytes / 8], caller
 *                  owned and kept between calls, 256-byte aligned; layout
 *                  [slot][batch * heads][64][blocks_per_frame][2]: channel
 *                  2c + e of the pooled key at block position p sits at
 *                  [c][p][e].
 *  other arguments as lcsa_select (the workspace holds the pooled Q).
 * Errors: as lcsa_select, plus INVALID (ring or new_frames out of range). */
lcsa_status lcsa_select_ring(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k_ring,
                             const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                             int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                             void* d_workspace, size_t workspace_bytes, void* stream);

/* Factored 3D rotary position embedding of Q and K, fused into selection.
 * The DiT turns its queries and keys with a factored 3D RoPE (NxDI FlashVSR
 * contrib page, "Model Information"), and that pass is part of the attention
 * glue around the sparse kernel (FlashVSR Hopper PR page, "What Was Actually
 * Slow"; "How I Fixed It" lists a coalesced RoPE kernel).  Here the pooling
 * pass of selection, which reads Q and K anyway, turns them, writes the
 * turned tensors and pools the turned values, so the separate read of Q and
 * K by a rotary pass goes away.
 * Channel pair j (channels 2j, 2j + 1, a complex number) turns by:
 *   j < pairs_t                      the row of table_t for the token's
 *                                    KV-window frame (a query of query frame
 *                                    tq is window frame kv_frames - q_frames
 *                                    + tq),
 *   pairs_t <= j < pairs_t + pairs_h the row of table_h for its token row,
 *   the rest                         the row of table_w for its token column.
 * Tables are float (cos, sin) pairs, row-major [position][pair][2]; the
 * caller chooses frequencies and the split (pairs_t + pairs_h + pairs_w =
 * head_dim / 2).  Each turned value x0 cos - x1 sin, x0 sin + x1 cos is
 * rounded once to bf16 (nearest, ties to even) from its exact value; pooling,
 * scores and the caller's later lcsa_attend on the outputs see exactly those
 * bf16 values. */
typedef struct lcsa_rope {
  int32_t pairs_t, pairs_h, pairs_w;
  int32_t reserved;              /* 0 */
  const float* table_t;          /* device float[kv_frames][pairs_t][2] */
  const float* table_h;          /* device float[grid_h][pairs_h][2] */
  const float* table_w;          /* device float[grid_w][pairs_w][2] */
} lcsa_rope;

/* lcsa_select on the turned Q and K, which it also writes out.
 *  q, k            unturned inputs, read only.
 *  rope            the tables (8-byte aligned device pointers).
 *  q_rot, k_rot    bf16 outputs of the shapes of q and k (own strides,
 *                  16-byte aligned); q_rot may be q itself and k_rot k
 *                  itself (each element is read and then written by the same
 *                  thread); otherwise they must not overlap each other or
 *                  the inputs.
 *  other arguments and the CSR result as lcsa_select; pass q_rot and k_rot
 *  to lcsa_attend.
 * Errors: as lcsa_select, plus NULL (rope or a table with pairs), INVALID
 * (pair counts), ALIGN (tables or outputs). */
lcsa_status lcsa_select_rope(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                             const lcsa_rope* rope, const lcsa_tensor* q_rot,
                             const lcsa_tensor* k_rot, int32_t* d_row_ptr, int32_t* d_col_idx,
                             double* d_scores, void* d_workspace, size_t workspace_bytes,
                             void* stream);

/* lcsa_select_ring with the rotary embedding: the new_frames newest window
 * frames of k_ring are turned, written to the same ring slots of k_rot_ring
 * (a ring of the same slots and strides rules) and pooled into d_kcache; the
 * cache entries of older frames must hold pooled turned keys (an earlier
 * call of this function).  Q is turned into q_rot.  table_t rows are
 * KV-window frames of this call.
 * Errors: as lcsa_select_ring and lcsa_select_rope. */
lcsa_status lcsa_select_ring_rope(lcsa_plan_t plan, const lcsa_tensor* q,
                                  const lcsa_tensor* k_ring, const lcsa_kv_ring* ring,
                                  int32_t new_frames, double* d_kcache, const lcsa_rope* rope,
                                  const lcsa_tensor* q_rot, const lcsa_tensor* k_rot_ring,
                                  int32_t* d_row_ptr, int32_t* d_col_idx, double* d_scores,
                                  void* d_workspace, size_t workspace_bytes, void* stream);

/* Steady threshold reuse.  On the FlashVSR Hopper PR page the last GH200
 * configuration stores each DiT block's mask threshold from a steady chunk
 * and applies it to later chunks in place of a new ranking
 * ("Remove the remaining control-plane tax"; quality-gated in "Recommended
 * GH200 Controls").  The page does not define the threshold; here it is
 * each CSR row's keep-th largest window score (keep = min(k, |window|)),
 * which with the same scores and no tie at that score selects exactly the
 * top-k.  A reused threshold selects by the new chunk's scores: the kept
 * count varies by row, from none to the whole window, so the result is an
 * approximation of top-k, not equal to it.
 *
 * Both calls take the forms of the selections above: ring == NULL reads k as
 * the contiguous window (new_frames and d_kcache ignored), otherwise as
 * lcsa_select_ring; rope == NULL takes q and k as already turned (q_rot and
 * k_rot ignored), otherwise as lcsa_select_rope / lcsa_select_ring_rope.
 *
 * lcsa_select_steady: the top-k selection of those forms (same CSR), plus
 *  d_kth           device double[rows], 8-byte aligned, written: row r's
 *                  keep-th largest window score (rows in CSR order).
 * Errors: as the form used, plus NULL (d_kth), ALIGN (d_kth). */
lcsa_status lcsa_select_steady(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                               const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                               const lcsa_rope* rope, const lcsa_tensor* q_rot,
                               const lcsa_tensor* k_rot, int32_t* d_row_ptr, int32_t* d_col_idx,
                               double* d_kth, double* d_scores, void* d_workspace,
                               size_t workspace_bytes, void* stream);

/* lcsa_select_reuse: selection by threshold instead of top-k.
 *  d_tau           device double[rows], 8-byte aligned, read: row r keeps
 *                  every window block whose float64 pooled score is >= d_tau[r]
 *                  (-inf keeps the whole window; +inf or NaN keeps nothing).
 *  d_row_ptr       device int32[rows + 1], written: r * max_window.
 *  d_col_idx       device int32[rows * max_window], written: row r's kept
 *                  blocks ascending, then -1 to the end of its max_window
 *                  entries.  Pass it to lcsa_attend / lcsa_attend_ring with
 *                  nnz = rows * max_window: attention skips -1 entries, and a
 *                  row that keeps nothing gives O = 0 and LSE = -inf.
 *  d_scores        as lcsa_select (the scores compared with d_tau).
 * Errors: as the form used, plus NULL (d_tau), ALIGN (d_tau), SHAPE
 * (rows * max_window >= 2^31). */
lcsa_status lcsa_select_reuse(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                              const lcsa_kv_ring* ring, int32_t new_frames, double* d_kcache,
                              const lcsa_rope* rope, const lcsa_tensor* q_rot,
                              const lcsa_tensor* k_rot, const double* d_tau, int32_t* d_row_ptr,
                              int32_t* d_col_idx, double* d_scores, void* d_workspace,
                              size_t workspace_bytes, void* stream);

/* Block-sparse attention with K and V read from a frame ring; otherwise as
 * lcsa_attend (same result as on the contiguous window).
 * Errors: as lcsa_attend, plus INVALID (ring out of range). */
lcsa_status lcsa_attend_ring(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k_ring,
                             const lcsa_tensor* v_ring, const lcsa_kv_ring* ring,
                             const int32_t* d_row_ptr, const int32_t* d_col_idx, int64_t nnz,
                             const lcsa_tensor* o, float* d_lse, void* d_workspace,
                             size_t workspace_bytes, void* stream);

/* Block-sparse attention for a CSR whose rows differ in length, such as the
 * output of lcsa_select_reuse (rows keep every block at or above a stored
 * threshold, so their lengths vary: the steady threshold reuse of the
 * FlashVSR Hopper PR page, "Remove the remaining control-plane tax"), or a
 * caller's mask.  Same result as lcsa_attend (ring == NULL) or
 * lcsa_attend_ring (ring given), to rounding: rows are taken longest first
 * instead of in the plan's visiting order, so that no long row starts last
 * and the rows split in the last, partly filled round are the shortest.  The
 * order is computed on the device from d_row_ptr / d_col_idx (two small
 * kernels before the attention kernel; stable, so every run takes the same
 * order and gives the same bits).
 *  k, v            the contiguous KV window (ring == NULL) or the rings.
 *  d_workspace     required, 256-byte aligned, at least
 *                  attend_workspace_bytes: the split pieces as in
 *                  lcsa_attend, then the row lengths and the row order.
 *  Other arguments as lcsa_attend.
 * Errors: as lcsa_attend (WORKSPACE for a NULL or short workspace), plus
 * INVALID (ring out of range). */
lcsa_status lcsa_attend_varlen(lcsa_plan_t plan, const lcsa_tensor* q, const lcsa_tensor* k,
                               const lcsa_tensor* v, const lcsa_kv_ring* ring,
                               const int32_t* d_row_ptr, const int32_t* d_col_idx, int64_t nnz,
                               const lcsa_tensor* o, float* d_lse, void* d_workspace,
                               size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* lcsa_status_string(lcsa_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* lcsa_last_error(void);

/* LCSA_ABI_VERSION of the loaded library. */
int32_t lcsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCSA_H_ */
