/*
 * swa.h - C ABI of the MI355X (gfx950) sliding-window FlashAttention library.
 *
 * Operation (forward): for every participating batch b and head n of a TND
 * packed batch,
 *     out = softmax(mask(scale * Q K^T)) V
 * with the saved row statistics softmax_max (row max of the scaled, masked
 * scores) and softmax_sum (sum of exp(score - softmax_max)).
 *   - formula: FlashAttentionVarLenScore API doc, "计算公式" (no pse, no
 *     dropout, keep_prob = 1, no explicit atten_mask tensor);
 *   - statistics: PyPTO-Gym FlashAttentionScoreGrad article, "前向公式" and
 *     "反向公式" (P = exp(QK^T*scale - softmax_max) / softmax_sum);
 *   - TND packing with cumulative per-batch ends: API doc, "算子功能" and
 *     parameters actualSeqQLenOptional / actualSeqKvLenOptional;
 *   - masks: op-plugin sliding-window blog, section 1.3 "SparseMode说明"
 *     (and explainer 6.6), with sequence-local indices i (query), j (key) of
 *     a batch with Sq queries and Skv keys:
 *       sparse_mode 0           no mask;
 *       sparse_mode 2 (LEFT_UP_CAUSAL)     keeps j <= i;
 *       sparse_mode 3 (RIGHT_DOWN_CAUSAL)  keeps j - i <= Skv - Sq;
 *       sparse_mode 4 (BAND)    keeps -pre_tokens <= j - i <= next_tokens.
 *
 * Operation (backward): aclnnFlashAttentionUnpaddingScoreGradV2 explainer,
 * sections 2.3 and 4.2, and the PyPTO-Gym article, "反向公式":
 *     P  = exp(scale Q K^T - softmax_max) / softmax_sum   (caller's stats)
 *     D  = rowsum(dY * out)                                (caller's out)
 *     dP = dY V^T,  dS = P * (dP - D)
 *     dV = P^T dY,  dQ = scale dS K,  dK = scale dS^T Q
 *
 * Call pattern: query the workspace size, let the caller allocate it on the
 * device, then call the operation on a stream (the two-phase pattern of the
 * aclnn APIs, explainer section 3).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   q, out, dy, dq     [t_q,  num_heads, head_dim]   element type `dtype`
 *   k, v, dk, dv       [t_kv, num_kv_heads, head_dim] element type `dtype`
 *                      (num_kv_heads = num_heads except in the *_ex calls)
 *   softmax_max/_sum   [t_q,  num_heads, 8] float32; all 8 entries of a row
 *                      hold the same value (TND statistics layout of the
 *                      explainer, section 4.2; column 0 is the one read).
 *   cu_seqlens_q/_kv   HOST int64 arrays of num_seqs inclusive cumulative
 *                      ends, no leading zero (e.g. {256}; {2, 5, 9, 0, 0}:
 *                      a zero after a positive entry starts a trailing run of
 *                      non-participating batches, explainer section 6.4).
 *
 * Conventions that the pages leave open:
 *   - a query row with no allowed key gets out = 0, softmax_max = -inf,
 *     softmax_sum = 0 and dq = 0; a key no query attends gets dk = dv = 0;
 *   - tokens after the last participating end get out = 0, softmax_max =
 *     -inf, softmax_sum = 0, dq = dk = dv = 0;
 *   - sparse_mode 0, 2 and 3 ignore pre_tokens / next_tokens;
 *   - the causal diagonal of modes 2 and 3 starts in the corner the name
 *     gives (top-left: j <= i; bottom-right: j - i <= Skv - Sq), so with
 *     Sq > Skv the first Sq - Skv rows of a mode-3 batch are empty.
 *
 * Ownership: every device buffer, the workspace included, belongs to the
 * caller; the library never allocates or frees caller memory.  Host arrays
 * are read during the call only.  All device work is enqueued on `stream`
 * (a hipStream_t; NULL = the default stream) and the calls return without
 * waiting for it; the caller keeps the buffers alive until the stream has
 * finished.  Calls on one stream are ordered; distinct calls that share a
 * workspace must not overlap in time.
 *
 * Errors: all validation runs on the host before anything is enqueued; on a
 * non-OK status nothing is written.  swa_last_error() returns a message for
 * the last non-OK status of the calling thread.
 */
#ifndef SWA_H_
#define SWA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swa_status {
  SWA_OK = 0,
  /* a required pointer is NULL (the pages' ACLNN_ERR_PARAM_NULLPTR, 161001) */
  SWA_ERR_NULLPTR = 1,
  /* an argument is out of range: sparse_mode not 0/2/3/4, sizes, inconsistent or
   * decreasing cumulative ends, pre_tokens + next_tokens < 0, non-finite
   * scale (the pages' ACLNN_ERR_PARAM_INVALID, 161002) */
  SWA_ERR_INVALID = 2,
  /* valid on the pages but not provided by this library: head_dim other than
   * 64 or 128, fp16, and sparse_mode 4 with a batch whose query and key
   * lengths differ */
  SWA_ERR_UNSUPPORTED = 3,
  /* workspace_bytes is smaller than the size query returned */
  SWA_ERR_WORKSPACE = 4,
  /* a HIP runtime call failed; the message carries hipGetErrorString */
  SWA_ERR_HIP = 5
} swa_status;

typedef enum swa_dtype {
  SWA_DTYPE_FP32 = 0,
  SWA_DTYPE_BF16 = 1,
  SWA_DTYPE_FP16 = 2 /* listed by the pages; returns SWA_ERR_UNSUPPORTED */
} swa_dtype;

/* Device workspace bytes that swa_forward needs for a batch of num_seqs
 * sequences (bounds only depend on the sizes, not on the lengths). */
swa_status swa_forward_workspace_size(int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                      int64_t num_heads, int64_t head_dim, int32_t dtype,
                                      size_t* bytes);

/* Device workspace bytes that swa_backward needs: the tile schedules and the
 * row terms D = rowsum(dY * out) (stored negated for bf16) and lse2, 8 bytes
 * per (token, head) of the queries beside the schedules. */
swa_status swa_backward_workspace_size(int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                       int64_t num_heads, int64_t head_dim, int32_t dtype,
                                       size_t* bytes);

/* Forward pass.  Writes out, softmax_max, softmax_sum.  `scale` is the
 * multiplier of Q K^T (usually head_dim^-0.5, API doc, scaleValueOptional).
 * Valid ranges: num_seqs 1..2048, t_q and t_kv 1..2^20, num_heads 1..256,
 * head_dim 1..768 (64 and 128 supported). */
swa_status swa_forward(const void* q, const void* k, const void* v,
                       const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                       int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                       int64_t head_dim, int32_t dtype, double scale, int64_t pre_tokens,
                       int64_t next_tokens, int64_t sparse_mode, void* out, float* softmax_max,
                       float* softmax_sum, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Backward pass.  Takes the forward's out and statistics verbatim (it does
 * not recompute them) and writes dq, dk, dv.  The sequence, shape and scalar
 * arguments must be those of the forward call that produced out and the
 * statistics; the library cannot check this.
 * Both input types run the two-pass structure of the PyPTO-Gym
 * FlashAttentionScoreGrad article (两趟循环结构): one kernel for dK/dV over
 * key blocks and one for dQ over query blocks, each recomputing P and dS, with
 * no atomics, so every output is bitwise reproducible (the deterministic mode
 * of the explainer, section 6.1).  bf16: the dQ kernel runs first and also
 * forms the row terms D and lse2 that the dK/dV kernel reads.  fp32: a
 * preprocess kernel forms the row terms, then the dK/dV and dQ kernels run. */
swa_status swa_backward(const void* q, const void* k, const void* v, const void* dy,
                        const void* out, const float* softmax_max, const float* softmax_sum,
                        const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                        int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                        int64_t head_dim, int32_t dtype, double scale, int64_t pre_tokens,
                        int64_t next_tokens, int64_t sparse_mode, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Extended calls: grouped key/value heads and dropout with a given mask.
 * swa_forward / swa_backward are these with num_kv_heads = num_heads and
 * drop_mask = NULL.  Every other argument, the workspace sizes included (they
 * take num_heads = the query head count), is as there.
 *
 * Grouped heads (GQA, explainer section 6.2): q, out, dy, dq and the
 * statistics have num_heads heads, k, v, dk and dv have num_kv_heads, and
 * num_heads must be a whole multiple G of num_kv_heads (else
 * SWA_ERR_INVALID).  Query head n reads key/value head n / G (integer
 * division); dk and dv of a key/value head sum the contributions of its G
 * query heads (inside one workgroup, so the bf16 backward stays
 * deterministic).
 *
 * Dropout (VarLenScore API doc, 计算公式: attention_out =
 * Dropout(softmax(...), keep_prob) * value; dropMaskOptional,
 * keepProbOptional; explainer section 6.3): drop_mask is DEVICE memory,
 * 4-byte aligned, holding one keep bit per (batch, query head, query row,
 * key): bit e is bit e % 8 (least significant first) of byte e / 8, and e
 * runs over the participating batches, then the heads, then the Sq x Skv
 * matrix of that batch and head row by row, so there are
 * sum_b num_heads * Sq_b * Skv_b bits; drop_mask_bytes must cover them
 * rounded up to whole 32-bit words (else SWA_ERR_INVALID).  A kept
 * probability is scaled by 1 / keep_prob (keep_prob in (0, 1], the fraction
 * of ones; else SWA_ERR_INVALID), a dropped one is zero; softmax_max /
 * softmax_sum are those of the undropped softmax.  The backward takes the
 * same mask and keep_prob.  drop_mask = NULL: no dropout (keep_prob and
 * drop_mask_bytes are ignored). */
swa_status swa_forward_ex(const void* q, const void* k, const void* v,
                          const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                          int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                          int64_t num_kv_heads, int64_t head_dim, int32_t dtype, double scale,
                          int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                          const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                          void* out, float* softmax_max, float* softmax_sum, void* workspace,
                          size_t workspace_bytes, void* stream);
swa_status swa_backward_ex(const void* q, const void* k, const void* v, const void* dy,
                           const void* out, const float* softmax_max, const float* softmax_sum,
                           const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                           int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                           int64_t num_kv_heads, int64_t head_dim, int32_t dtype, double scale,
                           int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                           const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                           void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * backward of swa_backward_ex with no workspace argument.  It calls no
 * hipMalloc, hipFree or other allocating routine; its schedule tables and
 * row terms live in a fixed scratch array of SWA_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds on each device it runs on until the
 * process ends.  A problem whose backward workspace (swa_backward_workspace_size)
 * exceeds that size returns SWA_ERR_WORKSPACE and writes nothing.  All calls
 * on one device share its scratch, which keeps the last call's contents:
 * calls that overlap in time on one device (on different streams, or from
 * several threads) race and must not be issued.  The schedule table is
 * copied from host memory with a synchronous copy, skipped when the device's
 * scratch already holds the same table.  Arguments, layouts, results and
 * every other status as in swa_backward_ex. */
#define SWA_NOALLOC_SCRATCH_BYTES (32u << 20)
swa_status swa_backward_noalloc(const void* q, const void* k, const void* v, const void* dy,
                                const void* out, const float* softmax_max,
                                const float* softmax_sum, const int64_t* cu_seqlens_q,
                                const int64_t* cu_seqlens_kv, int64_t num_seqs, int64_t t_q,
                                int64_t t_kv, int64_t num_heads, int64_t num_kv_heads,
                                int64_t head_dim, int32_t dtype, double scale,
                                int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                                const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                                void* dq, void* dk, void* dv, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* swa_last_error(void);

/* Host-only: the tile schedule the kernels would run, for checking the
 * skip pattern.  direction 0 = forward (items are query blocks, tiles are
 * key blocks), 1 = backward dK/dV (items are key blocks, tiles are query
 * blocks), 2 = backward dQ (items are query blocks, tiles are key blocks).
 * Writes rows of 4 int32 {sequence, item block, tile, kind} in schedule
 * order, kind 1 = partial (element mask applied), 2 = full (no mask); an
 * item with no visited tile contributes one row {sequence, block, -1, 0}.
 * rows_out may be NULL to query the count; *n_rows receives the number of
 * rows (at most `capacity` are written).  *block_item / *block_tile receive
 * the block sizes used. */
swa_status swa_debug_tile_schedule(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                   int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                   int64_t head_dim, int32_t dtype, int64_t pre_tokens,
                                   int64_t next_tokens, int64_t sparse_mode, int32_t direction,
                                   int32_t* rows_out, int64_t capacity, int64_t* n_rows,
                                   int32_t* block_item, int32_t* block_tile);

/* Device cache of tile schedules.  The library keeps device copies of the
 * schedules (the tile ranges and work lists its kernels read) of up to 64
 * recent problems per process, 256 MiB at most, keyed by the device, the
 * cumulative lengths and every size and mask argument; a call on a cached
 * problem neither rebuilds nor uploads its schedule.  An entry is written
 * once, by a synchronous copy, before any kernel reads it; evicting one waits
 * until its device is idle.  Host threads may call at once: an entry that a
 * call is using is evicted only after that call has enqueued its kernels.
 * Enabled by default; enable = 0 frees every entry (waiting for the devices
 * to be idle; an entry in use by a call on another thread is freed when that
 * call returns) and makes calls upload their schedule into the caller's
 * workspace instead, as swa_backward_noalloc always does into its scratch. */
swa_status swa_schedule_cache_enable(int32_t enable);

/* Kernel timing (instrumentation for benchmarks).  While enabled, every
 * kernel the library launches is bracketed by two HIP events recorded on its
 * stream.  swa_profile_read waits for the recorded launches of one kernel
 * kind, returns their summed duration (ms) and count, and forgets them.
 * Kernel kinds: 0 forward, 1 backward preprocess (fp32), 2 backward dK/dV,
 * 3 unused, 4 zero fill, 5 backward dQ (for bf16 with the row terms).  Not thread-safe across concurrent streams
 * (launches from all threads are pooled). */
swa_status swa_profile_enable(int32_t enable);
swa_status swa_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H_ */
