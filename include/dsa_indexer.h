/*
 * dsa_indexer.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention
 * lightning-indexer library (libdsa_indexer.so).
 *
 * The library scores, for every query token, each earlier cached token of a
 * paged FP8 indexer-K cache, selects the causal top-k token positions and
 * writes them into a shared int32 index buffer; IndexCache "S" layers reuse
 * the buffer written by the previous "F" layer of the same forward pass.
 *
 * Sources (web pages, cited by title and section):
 *  [KVB] GLM-5.3 inference pipeline (12): paging budget, prefix hits and
 *        eviction of the main KV and indexer caches -- byte accounts (132 B per
 *        token per layer: 128 FP8 key bytes + one fp32 scale per 128-element
 *        block), SGLang buffer shape (64-token pages of 8448 bytes), eviction
 *        (keys first, then scales, inside every page), top-k index buffer and
 *        logits budget (fp32 [rows, cols], rows aligned to 256 columns).
 *  [HBM] HBM index architecture design (vLLM research notes), sections 2.3
 *        and 4.2 -- block_table / positions / query_start_loc and
 *        slot = block_table[req, pos / 64] * 64 + pos % 64.
 *  [IC]  vLLM IndexCache practical guide -- section 2 (F/S layers, shared
 *        buffer, -1 clear, reuse within one pass), section 3 (index_topk_freq,
 *        index_topk_pattern, index_skip_topk_offset and the skip rule),
 *        section 4 (pattern semantics), section 5 item 3 (MTP layers).
 *  [RFC] RFC: DeepseekV32 model support (Ascend msmodeling), section 2.1.3 --
 *        the indexer path is FP8 (fp8_index operator).
 * The score (per-head dot product q_h . k_s, ReLU, per-head weighted sum) is
 * the lightning-indexer score of DeepSeek-V3.2 (arXiv:2512.02556, cited by
 * [KVB]); the pages print no formula for it.
 *
 * Conventions for every entry point:
 *  - Pointers documented "device" are device (HBM) addresses on the current
 *    HIP device; "host" pointers are ordinary host memory.
 *  - The caller owns every buffer.  No entry point allocates device memory;
 *    scratch comes from a caller-provided workspace sized by the *_size
 *    queries.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *    device work is enqueued asynchronously on it; nothing synchronises.
 *  - Return value: DSA_OK (0) or a negative dsa_status.  Argument errors are
 *    detected on the host before anything is enqueued; the message is
 *    available from dsa_last_error() on the calling thread.
 *  - Device-side range errors never fault; each raises a sticky flag,
 *    readable with dsa_device_error_flags().  A block_table entry outside
 *    the page pool: the logits of that page's tokens are -inf.  A position
 *    outside the logits row (p < 0 or p >= ld) or past the request's
 *    block-table row (p / 64 >= bt_stride): the row's logits are not
 *    written, and its top-k row (forward, run, or dsa_indexer_topk for p <
 *    0 or p >= ld) is all -1.
 *  - Supported shapes: head_dim == 128, page_size == 64, 1 <= H <= 64.
 *  - The *_workspace_size queries return 0 for arguments the matching entry
 *    point rejects or treats as a no-op (T <= 0, T > 2^31, ld <= 0,
 *    ld > 2^30, H outside [1, 64]); within those limits their sums cannot
 *    wrap.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad pattern, ...   */
  DSA_ERR_UNSUPPORTED = -2,   /* head_dim != 128, page_size != 64, H > 64   */
  DSA_ERR_WORKSPACE = -3,     /* workspace smaller than the size query      */
  DSA_ERR_HIP = -4            /* a HIP runtime call or launch failed        */
} dsa_status;

#define DSA_HEAD_DIM 128
#define DSA_PAGE_TOKENS 64
#define DSA_PAGE_BYTES 8448          /* 64 x 128 key bytes, then 64 x fp32  */
#define DSA_TOKEN_BYTES 132
#define DSA_LOGITS_ROW_ALIGN 256     /* ld % 256 == 0 ([KVB] logits budget) */
#define DSA_MAX_HEADS 64

/* Device error flags (dsa_device_error_flags). */
#define DSA_DEVERR_PAGE_OUT_OF_RANGE 1u
#define DSA_DEVERR_POSITION_OUT_OF_RANGE 2u

/* Message of the last failed call on this thread ("" if none). */
const char* dsa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int dsa_version(void);

/*
 * dsa_quantize_q -- per (token, head) FP8 quantisation of the indexer query
 * ([RFC] 2.1.3: FP8 indexer path; [KVB]: one fp32 scale per 128-element
 * block, the granularity the K cache uses).
 *   q_bf16   device, bf16 [T, H, 128], row-major, contiguous.
 *   q_fp8    device, out: OCP e4m3fn codes [T, H, 128].
 *   q_scale  device, out: fp32 [T, H].
 * Per 128-element block: amax = max|q|, s = amax / 448 (IEEE fp32 division;
 * s = 1 when amax == 0), code = e4m3fn(q / s) with IEEE fp32 division,
 * round-to-nearest-even and saturation to +-448.  T == 0 is a no-op.
 */
int dsa_quantize_q(const void* q_bf16, int64_t T, int H, int head_dim,
                   uint8_t* q_fp8, float* q_scale, void* stream);

/*
 * dsa_indexer_logits -- causal lightning-indexer logits over a paged FP8
 * indexer-K cache.
 *   q_fp8, q_scale   device, output of dsa_quantize_q: [T, H, 128], [T, H].
 *   weights          device, fp32 [T, H]: per (token, head) weight.
 *   k_cache          device, uint8 [num_pages, 8448]: page P holds the
 *                    e4m3fn keys of its 64 tokens (64 x 128 bytes) followed
 *                    by their 64 little-endian fp32 scales ([KVB]).
 *   block_table      device, int32 [R, bt_stride]: physical page of logical
 *                    page j of request r ([HBM] 2.3).
 *   query_start_loc  device, int32 [R + 1]: rows of request r are
 *                    [qsl[r], qsl[r+1]) ([HBM] 4.2).
 *   positions        device, int32 [T]: absolute position p_t of row t.
 *   logits           device, out: fp32 [T, ld], ld % 256 == 0 and
 *                    ld > every p_t.
 * Row t (request r, position p) gets, for every s <= p,
 *   logits[t, s] = sum_h w[t,h] * max(qhat[t,h,:] . khat[s,:], 0)
 * with qhat = code * q_scale and khat = code * k_scale, accumulated in fp32;
 * columns p < s < 64 * ceil((p+1)/64) are written as -inf; later columns are
 * not written.  Requires the block_table row to hold ceil((p+1)/64) valid
 * pages.  head_dim must be 128, page_size 64, 1 <= H <= 64.
 */
int dsa_indexer_logits(const uint8_t* q_fp8, const float* q_scale,
                       const float* weights, const uint8_t* k_cache,
                       int64_t num_pages, const int32_t* block_table,
                       int64_t bt_stride, const int32_t* query_start_loc,
                       const int32_t* positions, int64_t T, int R, int H,
                       int head_dim, int page_size, float* logits, int64_t ld,
                       void* stream);

/*
 * dsa_logits_schedule -- the decode page schedule of a batch, for
 * dsa_indexer_logits_scheduled: which wave scores which row's page range,
 * with the request and the first physical pages of each range resolved
 * through block_table ([HBM] 2.3, 4.2).  It depends only on block_table,
 * query_start_loc, positions, T, R and ld, so one schedule serves every
 * layer of a batch (the IndexCache F layers of a pass share them).  Built
 * only for batches of at most 128 rows (dsa_logits_schedule_size gives 0
 * otherwise: nothing to build, no error).
 *   schedule  device, out: dsa_logits_schedule_size(T, ld) bytes.
 * A position outside the logits or block-table row raises
 * DSA_DEVERR_POSITION_OUT_OF_RANGE and gives that row no range.
 */
size_t dsa_logits_schedule_size(int64_t T, int64_t ld);

int dsa_logits_schedule(const int32_t* block_table, int64_t bt_stride,
                        const int32_t* query_start_loc,
                        const int32_t* positions, int64_t T, int R,
                        int64_t ld, int32_t* schedule, size_t sched_bytes,
                        void* stream);

/*
 * dsa_indexer_logits_scheduled -- dsa_indexer_logits with a page schedule
 * built by dsa_logits_schedule for the same block_table, query_start_loc,
 * positions, T, R and ld (and the same dsa_set_option knobs), enqueued
 * before it: each decode wave then starts its K loads after one load of its
 * schedule entry.  Arguments and results as for dsa_indexer_logits, bit for
 * bit; schedule == NULL, or a batch the schedule does not serve (more than
 * 128 rows, rows sharing a request's keys), runs dsa_indexer_logits.
 */
int dsa_indexer_logits_scheduled(const uint8_t* q_fp8, const float* q_scale,
                                 const float* weights, const uint8_t* k_cache,
                                 int64_t num_pages, const int32_t* block_table,
                                 int64_t bt_stride,
                                 const int32_t* query_start_loc,
                                 const int32_t* positions, int64_t T, int R,
                                 int H, int head_dim, int page_size,
                                 float* logits, int64_t ld,
                                 const int32_t* schedule, void* stream);

/*
 * dsa_indexer_topk -- per-row causal top-k into the shared index buffer
 * ([IC] 2: rows cleared to -1, then the top-k scattered in; [KVB] top-k
 * buffer: int32 [max_num_batched_tokens, index_topk]).
 *   logits     device, fp32 [T, ld]; row t reads columns 0..p_t only.
 *   positions  device, int32 [T].
 *   out        device, out: int32 [T, out_ld], out_ld >= k; slots [0, k) of
 *              every row are written.
 * n = p_t + 1 (n = 0, a row of -1, when p_t < 0 or p_t >= ld: a position
 * the logits call does not score).  If n <= k the row is 0, 1, ..., n-1
 * followed by -1.
 * Otherwise it holds the k token positions with the largest logits, ties at
 * the k-th value broken toward the lower position, listed in ascending
 * position order.  workspace/ws_bytes: dsa_topk_workspace_size() bytes of
 * device memory (may be 0 / NULL when that size is 0).
 */
int dsa_indexer_topk(const float* logits, int64_t ld, const int32_t* positions,
                     int64_t T, int k, int32_t* out, int64_t out_ld,
                     void* workspace, size_t ws_bytes, void* stream);

size_t dsa_topk_workspace_size(int64_t T, int64_t ld, int k);

/*
 * dsa_indexer_forward -- the whole indexer hot path of one layer for one
 * batch: dsa_quantize_q, dsa_indexer_logits and dsa_indexer_topk in one
 * call, with the same arguments, layouts and results (logits are written to
 * `logits` as by dsa_indexer_logits, the top-k rows to `out` as by
 * dsa_indexer_topk; [KVB], [HBM] 2.3 and 4.2, [IC] 2).
 *   q_bf16     device, bf16 [T, H, 128].
 *   workspace  device, dsa_forward_workspace_size(T, H, ld, k) bytes (q
 *              codes and scales, top-k scratch); contents on entry do not
 *              matter.
 * The three kernels run in turn on `stream` (a decode batch of at most 128
 * rows builds its page schedule in the quantisation launch, as
 * dsa_logits_schedule would, and scores with it); the result equals the
 * three separate calls bit for bit, except that a row whose position is past
 * its
 * block-table row (p / 64 >= bt_stride; flagged, logits not written) gets a
 * top-k row of -1.
 */
int dsa_indexer_forward(const void* q_bf16, const float* weights,
                        const uint8_t* k_cache, int64_t num_pages,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* query_start_loc,
                        const int32_t* positions, int64_t T, int R, int H,
                        int head_dim, int page_size, float* logits,
                        int64_t ld, int k, int32_t* out, int64_t out_ld,
                        void* workspace, size_t ws_bytes, void* stream);

size_t dsa_forward_workspace_size(int64_t T, int H, int64_t ld, int k);

/*
 * dsa_indexer_forward_noalloc -- dsa_indexer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (without the workspace),
 * same kernels, same results bit for bit.  Its scratch (q codes and scales,
 * top-k scratch) is one fixed array of DSA_NOALLOC_SCRATCH_BYTES inside the
 * library per device, held from the first call on that device until the
 * process ends; nothing in it needs to start at zero.  A batch whose
 * dsa_forward_workspace_size(T, H, ld, k) exceeds that limit is rejected
 * with DSA_ERR_WORKSPACE before anything is enqueued (for example the
 * 8192-row prefill chunk at H = 64: use dsa_indexer_forward).  Allocates
 * nothing and calls no allocating routine.  Every call on a device uses that
 * device's one array: calls that overlap on one device (two streams, or two
 * threads without ordering) race and give undefined results.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int dsa_indexer_forward_noalloc(const void* q_bf16, const float* weights,
                                const uint8_t* k_cache, int64_t num_pages,
                                const int32_t* block_table, int64_t bt_stride,
                                const int32_t* query_start_loc,
                                const int32_t* positions, int64_t T, int R,
                                int H, int head_dim, int page_size,
                                float* logits, int64_t ld, int k, int32_t* out,
                                int64_t out_ld, void* stream);

/*
 * dsa_logits_budget_bytes -- the logits memory budget ([KVB] section on
 * SGLang's logits budget): 30 % of the device's total_mem bytes; when a
 * static memory fraction is set (mem_fraction_static >= 0; pass a negative
 * value for none), the smaller of that and free_mem_fraction of the memory
 * outside the static part; free_mem_fraction is clamped to [0, 1].  At
 * least 1.  Host only.
 */
size_t dsa_logits_budget_bytes(size_t total_mem, double mem_fraction_static,
                               double free_mem_fraction);

/*
 * dsa_logits_chunk_rows -- query rows per scoring pass under a logits
 * budget ([KVB], same section): all T rows when T * ld fp32 elements are
 * under 8,000,000 or fit budget_bytes; otherwise budget_bytes / (ld * 4)
 * rows, at least 1.  0 for T <= 0 or ld <= 0.  Host only.
 */
int64_t dsa_logits_chunk_rows(int64_t T, int64_t ld, size_t budget_bytes);

/*
 * dsa_indexer_forward_chunked -- the forward pass with its logits bounded
 * by a budget ([KVB], SGLang logits budget: over the budget the query rows
 * are cut into pieces, each scored and ranked on its own, and the results
 * put together).  Arguments as for dsa_indexer_forward, except:
 *   (no logits argument) the logits of one chunk live in the workspace;
 *   rows_per_chunk  >= 1 (dsa_logits_chunk_rows gives the budget's);
 *   workspace       device, dsa_forward_chunked_workspace_size(T, R, H, ld,
 *                   k, rows_per_chunk) bytes: q codes and scales of all rows,
 *                   logits of rows_per_chunk rows, the chunk's rebased
 *                   query_start_loc, top-k scratch.
 * q is quantised once; then for each chunk [a, a + n) one small kernel
 * rebases query_start_loc to the chunk's rows, the logits of the chunk's
 * rows are scored into the workspace with the kernel class the whole batch
 * would use, and their top-k is written to out rows a .. a + n - 1.  out
 * equals dsa_indexer_forward's bit for bit, whatever rows_per_chunk.
 * Errors as for dsa_indexer_forward; also DSA_ERR_INVALID_ARG for
 * rows_per_chunk < 1 and DSA_ERR_WORKSPACE for a smaller workspace.
 */
int dsa_indexer_forward_chunked(const void* q_bf16, const float* weights,
                                const uint8_t* k_cache, int64_t num_pages,
                                const int32_t* block_table, int64_t bt_stride,
                                const int32_t* query_start_loc,
                                const int32_t* positions, int64_t T, int R,
                                int H, int head_dim, int page_size, int64_t ld,
                                int k, int32_t* out, int64_t out_ld,
                                int64_t rows_per_chunk, void* workspace,
                                size_t ws_bytes, void* stream);

size_t dsa_forward_chunked_workspace_size(int64_t T, int R, int H, int64_t ld,
                                          int k, int64_t rows_per_chunk);

/*
 * dsa_indexer_forward_fused -- the forward pass without a logits buffer
 * ([KVB], SGLang logits budget: the fp32 score buffer of rows x columns that
 * the budget bounds is never written; the context is cut into page splits,
 * each keeps only its candidates for the row's top-k, and the candidates
 * are merged and ranked).  Arguments as for dsa_indexer_forward, except:
 *   (no logits argument)
 *   workspace  device, dsa_forward_fused_workspace_size(T, R, H, ld, k)
 *              bytes; contents on entry do not matter.
 * A tiled batch (T > 2 R: prefill chunks, query rows over long contexts) is
 * scored twice by the default tiled kernel: once over every 32nd page (the
 * fused_sample_stride option: 16, 32 or 64; sparser when a row would have
 * more than 256 sampled pages), whose logits give each
 * row a lower bound of its k-th largest logit, then over every page, keeping
 * only the (logit, position) pairs at or above that bound, per row and page
 * split in position order.  The row's top-k is then selected from those
 * pairs.  When they cannot hold the answer (fewer than k, a split's slot
 * full, more than 16384), the row is scored again whole, with the same
 * arithmetic, into a scratch row of the workspace, and ranked from there.
 * Either way out holds exactly the top-k of the logits the default tiled
 * kernel computes: dsa_indexer_forward's rows bit for bit, when that call
 * uses the default kernel for the batch.  Other batches (T <= 2 R) run
 * dsa_indexer_forward with the logits in the workspace.  Errors as for
 * dsa_indexer_forward; DSA_ERR_UNSUPPORTED when the tile_pages_per_split
 * option cuts the pages into more splits than the workspace was sized for.
 * Rows outside query_start_loc's rows get -1.
 */
int dsa_indexer_forward_fused(const void* q_bf16, const float* weights,
                              const uint8_t* k_cache, int64_t num_pages,
                              const int32_t* block_table, int64_t bt_stride,
                              const int32_t* query_start_loc,
                              const int32_t* positions, int64_t T, int R,
                              int H, int head_dim, int page_size, int64_t ld,
                              int k, int32_t* out, int64_t out_ld,
                              void* workspace, size_t ws_bytes, void* stream);

size_t dsa_forward_fused_workspace_size(int64_t T, int R, int H, int64_t ld,
                                        int k);

/*
 * dsa_index_cache_mask -- IndexCache layer rule ([IC] 3, 4, 5.3), host only.
 *   pattern            host, nullable: one 'F'/'S' per DSA layer; overrides
 *                      freq when non-NULL; layers past its end are F.
 *   freq               index_topk_freq >= 1 (1 = every layer computes).
 *   offset             index_skip_topk_offset (the pages' default is 2).
 *   first_layer        layer id of is_skip[0] (0 for a trunk pass; the
 *                      first MTP layer's id for a draft pass), >= 0.
 *   num_hidden_layers  layers >= this are MTP/nextn layers; a negative
 *                      value means there are none.
 *   mtp_draft_step     draft step of the pass (0 = the step that computes).
 *   mtp_reuse          nonzero when index_share_for_mtp_iteration is on and
 *                      each draft position has one token (eagle topk 1;
 *                      [KVB] engineering judgement, item 4).
 *   is_skip            host, out: uint8 [num_layers], 1 = S (reuse), 0 = F.
 * Layer l = first_layer + i.  An MTP layer is S iff mtp_reuse and
 * mtp_draft_step > 0 ([IC] 5 item 3: full indexer, computes at draft step
 * 0, the runtime switch turns on reuse).  Otherwise, with a pattern: S iff
 * l < strlen(pattern) and pattern[l] == 'S'; without: S iff max(l - offset
 * + 1, 0) % freq != 0.  A pattern character other than 'F' or 'S' is an
 * error.
 */
int dsa_index_cache_mask(const char* pattern, int freq, int offset,
                         int first_layer, int num_layers,
                         int num_hidden_layers, int mtp_draft_step,
                         int mtp_reuse, uint8_t* is_skip);

/* Per-layer inputs of dsa_index_cache_run (ignored for S layers). */
typedef struct {
  const void* q_bf16;      /* device, bf16 [T, H, 128]                     */
  const float* weights;    /* device, fp32 [T, H]                          */
  const uint8_t* k_cache;  /* device, uint8 [num_pages, 8448]              */
  int64_t num_pages;
} dsa_layer_inputs;

/* Called on the calling thread after the work of layer id `layer`
 * (first_layer + its index) is enqueued on the stream (work the callback
 * enqueues on the same stream runs after it). */
typedef void (*dsa_layer_callback)(int layer, int is_full,
                                   int32_t* topk_buffer, void* user);

/*
 * dsa_index_cache_run -- one forward pass over a stack of DSA layers ([IC] 2).
 * F layers quantise q, score and write the top-k of rows [0, T) into
 * topk_buffer (int32 [buffer_rows, k], device); S layers enqueue nothing and
 * leave the buffer as the previous F layer wrote it.  layers[i] (host array
 * of num_layers entries) holds the inputs of layer id first_layer + i;
 * block_table, query_start_loc and positions (device) are shared by all
 * layers.  pattern .. mtp_reuse: the rule of dsa_index_cache_mask.
 *   snapshots    device, nullable: int32 [num_layers, T, k]; after layer i
 *                rows [0, T) of the buffer are copied to snapshots[i].
 *   is_skip_out  host, nullable: uint8 [num_layers], the mask used.
 *   cb, cb_user  nullable per-layer callback.
 *   rows_per_chunk  0 (or >= T): F layers run as dsa_indexer_forward with
 *                the logits of all T rows in the workspace; otherwise as
 *                dsa_indexer_forward_chunked with chunks of this many rows
 *                (the logits budget; same top-k rows bit for bit).
 *   workspace    device, dsa_run_workspace_size(T, R, H, ld, k,
 *                rows_per_chunk) bytes.
 * Rejects (DSA_ERR_INVALID_ARG) a mask whose first layer is S ([IC] 5.3:
 * it would read a buffer no layer has written in this pass), except in an
 * MTP draft pass that reuses (first_layer >= num_hidden_layers >= 0,
 * mtp_reuse, mtp_draft_step > 0): the buffer then holds the rows that draft
 * step 0 wrote, which the caller keeps between the passes.
 */
int dsa_index_cache_run(const char* pattern, int freq, int offset,
                        int first_layer, int num_layers,
                        int num_hidden_layers, int mtp_draft_step,
                        int mtp_reuse, const dsa_layer_inputs* layers,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* query_start_loc,
                        const int32_t* positions, int64_t T, int R, int H,
                        int64_t ld, int k, int64_t rows_per_chunk,
                        int32_t* topk_buffer, int64_t buffer_rows,
                        int32_t* snapshots, uint8_t* is_skip_out,
                        dsa_layer_callback cb, void* cb_user, void* workspace,
                        size_t ws_bytes, void* stream);

size_t dsa_run_workspace_size(int64_t T, int R, int H, int64_t ld, int k,
                              int64_t rows_per_chunk);

/*
 * dsa_slot_mapping -- physical cache slot of every query row's token
 * ([HBM] 2.3: slot = block_table[r, p / 64] * 64 + p % 64, r the request
 * of row t from query_start_loc).
 *   block_table      device, int32 [R, bt_stride].
 *   query_start_loc  device, int32 [R + 1], non-decreasing.
 *   positions        device, int32 [T].
 *   slots            device, out: int64 [T]; -1 where p < 0, p / 64 >=
 *                    bt_stride or the block-table entry is negative.
 * The slots are what dsa_indexer_k_write takes.  T == 0 is a no-op.
 */
int dsa_slot_mapping(const int32_t* block_table, int64_t bt_stride,
                     const int32_t* query_start_loc, int R,
                     const int32_t* positions, int64_t T, int64_t* slots,
                     void* stream);

/*
 * dsa_compressed_slot_mapping -- slots of a compressed cache ([HBM] 5.1,
 * 5.2, DeepSeek-V4): only a token whose position p has (p + 1) %
 * compress_ratio == 0 gets a slot; it is entry c = p / compress_ratio of its
 * request, stored at block_table[r, c / block_size] * block_size + c %
 * block_size.  block_size is the entries per storage block, the host
 * block's tokens / compress_ratio (256 / 4 = 64: the 64-entry, 8448-byte
 * page of dsa_indexer_k_write and dsa_indexer_logits).
 *   block_table, query_start_loc, positions  as for dsa_slot_mapping.
 *   slots        device, out: int64 [T]; -1 for a non-boundary token, p <
 *                0, c / block_size >= bt_stride or a negative entry.
 *   positions_c  device, out, nullable: int32 [T], the row's position in
 *                the compressed cache, (p + 1) / compress_ratio - 1 (the
 *                last entry whose tokens are all at or before p; -1 when
 *                none is, or p < 0) -- the positions dsa_indexer_logits
 *                and dsa_indexer_topk take over a compressed cache (a row
 *                with -1 sees no entry and is left out of those calls:
 *                the logits kernel flags a negative position).
 * compress_ratio 1 with block_size 64 equals dsa_slot_mapping.  Rejects
 * compress_ratio < 1 or block_size < 1.  T == 0 is a no-op.
 */
int dsa_compressed_slot_mapping(const int32_t* block_table,
                                int64_t bt_stride,
                                const int32_t* query_start_loc, int R,
                                const int32_t* positions, int64_t T,
                                int compress_ratio, int block_size,
                                int64_t* slots, int32_t* positions_c,
                                void* stream);

/*
 * dsa_indexer_k_write -- the indexer-K write path: quantise N new keys and
 * store each at its slot of the paged cache ([KVB] section on the indexer
 * cache's write path: FP8 key and FP32 scale at the token's in-page
 * offset; page layout as for dsa_indexer_logits).
 *   k_bf16        device, bf16 [N, 128], contiguous.
 *   slot_mapping  device, int64 [N]: slot of token i (page slot / 64, row
 *                 slot % 64); a negative slot writes nothing (padding).
 *   k_cache       device, in/out: uint8 [num_pages, 8448].
 * Per token: amax = max|k|, s = amax / 448 (IEEE fp32 division), code =
 * e4m3fn(k / s) (IEEE division, round to nearest even, saturating at 448);
 * an all-zero key stores s = 0 and zero codes.  Key bytes go to page * 8448
 * + row * 128, the scale to page * 8448 + 8192 + row * 4.  A slot >=
 * num_pages * 64 writes nothing and raises DSA_DEVERR_PAGE_OUT_OF_RANGE.
 * Two tokens with the same slot in one call: unspecified which is stored.
 */
int dsa_indexer_k_write(const void* k_bf16, int64_t N, int head_dim,
                        const int64_t* slot_mapping, uint8_t* k_cache,
                        int64_t num_pages, void* stream);

/*
 * dsa_topk_to_slots -- the sparse-attention hand-off in slot form: every
 * entry of the top-k rows (logical positions, as dsa_indexer_topk writes
 * them) as the physical cache slot of that token ([HBM] 2.3: block_table[r,
 * s / 64] * 64 + s % 64, r the request of the row) -- the slot the write
 * path stored its key at.
 *   topk         device, int32 [T, topk_ld], k entries used per row.
 *   block_table  device, int32 [R, bt_stride]; query_start_loc int32 [R+1].
 *   slots        device, out: int64 [T, k] (row stride k); -1 for a -1
 *                entry or an index without a block-table page.
 * DSA_ERR_INVALID_ARG unless T >= 0, k >= 1, topk_ld >= k, R >= 1 and
 * bt_stride >= 1, or for a null pointer when T > 0; T == 0 is a no-op.
 */
int dsa_topk_to_slots(const int32_t* topk, int64_t T, int k, int64_t topk_ld,
                      const int32_t* block_table, int64_t bt_stride,
                      const int32_t* query_start_loc, int R, int64_t* slots,
                      void* stream);

/*
 * dsa_topk_mask -- the sparse-attention hand-off in mask form ([RFC] 2.1.3,
 * sparse MLA: a tensor of the score's shape with 0 at the selected tokens
 * and -inf elsewhere, added to q k^T).
 *   topk  device, int32 [T, topk_ld], k entries used per row (-1 ignored).
 *   mask  device, out: fp32 [T, ld], ld % 256 == 0; every column written:
 *         0 if the row selects it, -inf otherwise (indices >= ld ignored).
 * The mask is written with non-temporal stores.  DSA_ERR_INVALID_ARG
 * unless T >= 0, k >= 1, topk_ld >= k and ld is a positive multiple of
 * 256, or for a null pointer when T > 0; T == 0 is a no-op.
 */
int dsa_topk_mask(const int32_t* topk, int64_t T, int k, int64_t topk_ld,
                  float* mask, int64_t ld, void* stream);

/*
 * dsa_device_error_flags -- sticky device-side range-error flags
 * (DSA_DEVERR_*) raised since the last reset; synchronises the device.
 * reset != 0 clears them.  Returns the flags, or a negative dsa_status.
 */
int dsa_device_error_flags(int reset);

/*
 * dsa_fp8_mfma_rate_probe -- measurement helper, not a step of the hot
 * path: enqueues on `stream` one launch in which every wave (two per SIMD)
 * runs `iters` rounds of 8 independent 16x16x128 FP8 MFMAs on register
 * operands -- no memory traffic -- and stores in *flops the FP8 operations
 * that launch performs.  Timed by the caller (events on the same stream), it
 * gives the FP8 matrix rate this device reaches at the clock it holds under
 * such a load, the measured counterpart of the published dense peak that
 * the logits kernels' rate is read against.  iters in [1, 1 << 24];
 * DSA_ERR_INVALID_ARG otherwise or for flops == NULL.
 */
int dsa_fp8_mfma_rate_probe(int iters, double* flops, void* stream);

/*
 * dsa_page_read_probe -- measurement helper, not a step of the hot path:
 * enqueues on `stream` one launch that reads the n K pages whose ids are
 * page_ids[0 .. n) (device, int32) from k_cache (device, [num_pages, 8448]
 * bytes, the layout of [KVB] SGLang buffer shape) whole -- 8 KB of keys and
 * 256 B of scales each, in 1 KB contiguous loads, three pages per wave --
 * and does nothing with the bytes.  Timed by the caller (events on the same
 * stream) over the pages a decode batch's rows reach, it gives the time a
 * bare read of exactly the bytes the decode logits kernel reads takes on
 * this device, with no metadata lookups and no compute: the attainable
 * floor that kernel's time is read against.  An id outside [0, num_pages)
 * reads nothing.  Errors: DSA_ERR_INVALID_ARG for n < 0, num_pages < 1 or a
 * null pointer with n > 0; DSA_ERR_UNSUPPORTED for n > 2^31.
 */
int dsa_page_read_probe(const uint8_t* k_cache, int64_t num_pages,
                        const int32_t* page_ids, int64_t n, void* stream);

/*
 * dsa_fp8_code_check -- check helper, not a step of the hot path: enqueues
 * on `stream` an exhaustive check of the FP8 arithmetic dsa_quantize_q's
 * fast path uses for a finite block with scale s = amax / 448 >= 2^-100
 * (the q quantisation's e4m3fn code of fp32(q / s), [RFC] 2.1.3 FP8
 * indexer) and writes three mismatch counts to counts (device, uint64 [3],
 * zeroed first): [0] fp32 values with |x| < 464 whose hardware e4m3
 * conversion differs from the library's integer round-to-nearest-even
 * encoder; [1] bf16 pairs (q, amax) with amax finite and positive, |q| <=
 * amax and s >= 2^-100 whose reciprocal-with-one-FMA quotient differs from
 * the IEEE quotient; [2] such pairs whose hardware code of that quotient
 * differs from the integer code of the IEEE quotient.  [2] == 0 is what the
 * fast path needs.  About 6.6 G cases; a few milliseconds.
 * DSA_ERR_INVALID_ARG for counts == NULL.
 */
int dsa_fp8_code_check(uint64_t* counts, void* stream);

/*
 * dsa_set_option -- tuning/testing knobs; returns the previous value or
 * DSA_ERR_INVALID_ARG for an unknown key or value.  Knobs are kept per
 * device (the calling thread's current HIP device) in atomics: concurrent
 * calls are safe, and each launch reads one snapshot of its device's knobs.
 * Value 0 restores the automatic choice.  Keys: "logits_kernel" (1
 * row-wise, 2 tiled with 8 waves x 2 rows, 3 tiled with direct loads, 4
 * row-wise on a (row, page group) grid, 5 tiled with 16 waves x 1 row but
 * ReLU as an add and an FMA per MFMA output instead of the default's shared
 * linear term, 6 the default tiled kernel whatever the batch's shape),
 * "row_pages_per_wave", "row_head_waves" (decode rows: 1 + the
 * waves per row that take its first pages before the positions are read;
 * default one such wave, 1 = none), "tile_pages_per_split",
 * "tile_pages_per_step" (16-row tile kernel: pages staged per copy step, 2
 * or 4; automatic: 4 when its grid takes more than two rounds of the
 * compute units), "topk_kernel" (rows of up to 49152 columns, keys in
 * registers: by default one 1024-thread workgroup per row, two 512-thread
 * workgroups per compute unit when the rows outnumber the compute units; 1
 * always the former, 4 always the latter; 2 keys cached in LDS; rows longer
 * than 65536 columns: 3 multi-workgroup radix select instead of sample
 * select), and for dsa_indexer_forward_fused "fused_sample_stride" (sample
 * every 16th, 32nd or 64th page, default 32; more sparsely when a row would
 * have more than 256 sampled pages), "fused_cand_cap" (n: at most n candidates per
 * row and page split; rows that overflow are re-scored),
 * "fused_force_rescue" (1: every row of more than k columns is re-scored;
 * the result must not change) and "fused_select" (candidate selection: 1
 * or 2 one wave per row with up to 4096 / 5120 candidates, when the batch
 * has at most 16 page splits per tile; 3 one 1024-thread workgroup per
 * row).
 */
int dsa_set_option(const char* key, int value);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
