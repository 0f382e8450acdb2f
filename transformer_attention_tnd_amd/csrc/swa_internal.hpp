// Internal declarations shared by the host side (validation, tile schedule,
// C ABI) and the HIP kernels.  Nothing here is part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/swa.h"

namespace swa {

// Block sizes.  Forward: a work item is one block of FWD_BM = 2 x FWD_HALF
// query rows of one sequence (one workgroup per item and head, two wave
// groups of FWD_HALF rows); it walks key tiles of FWD_BN.  Backward dK/dV: an
// item is one block of BWD_BN keys; it walks query tiles of BWD_BM rows.
// Backward dQ: an item is one block of DQ_BM query rows; it walks key tiles
// of FWD_BN.
constexpr int FWD_HALF = 128;
constexpr int FWD_BM = 2 * FWD_HALF;
constexpr int FWD_BN = 64;
constexpr int BWD_BN = 128;
constexpr int BWD_BM = 64;
constexpr int DQ_BM = FWD_HALF;

// One schedule entry (64 bytes, uploaded to the workspace).
//   tiles[i] = lo | hi << 16 : visited tile range [lo, hi] (empty if lo > hi)
//   full[i]  = flo | fhi << 16 : tiles in [flo, fhi] need no element mask
//   band     = {pre, next} of the sequence's mask (key j allowed for query i
//              iff -pre <= j - i <= next), clamped to +-2^30; unused when the
//              kernel's mode is 0 (no mask)
//   drop_base = first dropout-mask bit of the sequence (its head 0); head n
//              starts n * sq * skv bits later
// Forward items carry one range per FWD_HALF-row half (index 0, 1); backward
// items (dK/dV and dQ) use index 0 only.
struct Item {
  int32_t q_base;   // first token of the sequence in the query tensor
  int32_t kv_base;  // first token of the sequence in the key/value tensors
  int32_t sq;       // query length of the sequence
  int32_t skv;      // key/value length of the sequence
  int32_t block;    // item block index inside the sequence
  int32_t seq;      // batch index (diagnostics only)
  int32_t tiles[2];
  int32_t full[2];
  int32_t band[2];
  int64_t drop_base;
  int64_t pad;
};
static_assert(sizeof(Item) == 64, "Item layout");

inline int32_t pack_range(int64_t lo, int64_t hi) {
  if (lo > hi) { lo = 1; hi = 0; }
  return static_cast<int32_t>((lo & 0xffff) | ((hi & 0xffff) << 16));
}

struct Problem {
  int64_t num_seqs, t_q, t_kv, num_heads, num_kv_heads, head_dim;
  int32_t dtype;
  double scale;
  int64_t pre_tokens, next_tokens, sparse_mode;
  const int64_t* cu_q;
  const int64_t* cu_kv;
  const void* drop_mask;   // packed keep bits (null: no dropout)
  size_t drop_mask_bytes;
  double keep_prob;
};

// Persistent kernels: at most this many workgroups (one per compute unit);
// work list codes are item | head << 16.
constexpr int kMaxGrid = 1024;
inline int32_t work_code(int64_t item, int64_t head) {
  return static_cast<int32_t>(item | (head << 16));
}

// Dropout operands of the kernels: the packed keep bits as 32-bit words
// (null: no dropout), their count, 1 / keep_prob and log2(keep_prob).
struct DropArgs {
  const uint32_t* words;
  int64_t n_words;
  float rkp;
  float log2kp;
};

// Kernel arguments.  Element pointers are typeless; the kernels cast.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* smax;
  float* ssum;
  const Item* items;
  int32_t n_items;
  // persistent: workgroup w runs the units work[work_off[w] .. work_off[w + 1])
  // (codes item | head << 16) in order
  const int32_t* work;
  const int32_t* work_off;
  int32_t n_wg;
  int32_t num_heads;     // query heads (q, out, statistics)
  int32_t num_kv_heads;  // key/value heads; query head n reads head n / (num_heads / num_kv_heads)
  float scale_log2;  // scale * log2(e)
  int32_t mode;      // 0: no mask; otherwise each item's band applies
  DropArgs drop;
};

struct BwdPreArgs {
  const void* dy;
  const void* out;
  const float* smax;
  const float* ssum;
  float* drow;   // [N, t_q] rowsum(dY * out)
  float* lse2;   // [N, t_q] softmax_max*log2(e) + log2(softmax_sum), +inf if empty
  int64_t rows;  // t_q * N
  int32_t num_heads;
  int32_t t_q;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dy;
  float* drow;        // [N, t_q]: D = rowsum(dY o O) (fp32: from the preprocess
                      // kernel); -D, with dropout -D keep_prob (bf16: written by the dQ
                      // kernel, read by the dK/dV kernel)
  float* lse2;        // [N, t_q]: softmax_max log2(e) + log2(softmax_sum) (bf16 with
                      // dropout: + log2(keep_prob), so that exp2(s c - lse2) = P / keep_prob)
  // bf16 two-pass: the dQ kernel (launched first) computes D and lse2 of its
  // rows from out and the statistics and stores them for the dK/dV kernel
  const void* out;    // [t_q, N, D]
  const float* smax;  // [t_q, N, 8]
  const float* ssum;  // [t_q, N, 8]
  void* dq;           // dQ kernels only
  void* dk;
  void* dv;
  const Item* items;
  int32_t n_items;
  // persistent bf16 kernels: workgroup w runs the units
  // work[work_off[w] .. work_off[w + 1]) (codes item | head << 16) in order
  const int32_t* work;
  const int32_t* work_off;
  int32_t n_wg;          // persistent grid size
  int32_t num_heads;     // query heads (q, dy, dq, D, lse2)
  int32_t num_kv_heads;  // key/value heads (k, v, dk, dv); the dK/dV grid runs over these
  int32_t t_q;
  float scale;
  float scale_log2;
  int32_t mode;  // 0: no mask; otherwise each item's band applies
  DropArgs drop;
};

// Zero-fill of rows [row0, row1) of a [rows, N, D] tensor and, if smax is
// given, softmax_max = -inf / softmax_sum = 0 for those rows.
struct FillArgs {
  void* x;
  int64_t elem_bytes;
  int64_t row_elems;  // N * D
  int64_t row0, row1;
  float* smax;
  float* ssum;
  int64_t stat_row;   // N * 8
};

// Launchers (defined in the .hip files).  They return a hipError_t as int.
int launch_forward(const FwdArgs& a, int dtype, int head_dim, void* stream);
// fp32 only: D and lse2 of every row
int launch_bwd_pre(const BwdPreArgs& a, int head_dim, void* stream);
// the dK/dV kernel of either type over the dK/dV schedule (writes dk, dv)
int launch_backward(const BwdArgs& a, int dtype, int head_dim, void* stream);
// bf16 only: the dK/dV kernel over the dK/dV schedule (writes dk, dv);
// grouped key/value heads go to launch_bwd_kv_grouped
int launch_bwd_kv(const BwdArgs& a, int head_dim, void* stream);
int launch_bwd_kv_grouped(const BwdArgs& a, int head_dim, void* stream);
int launch_bwd_kv_grouped_drop(const BwdArgs& a, int head_dim, void* stream);
// bf16 only: the dQ kernel over the dQ schedule (writes dq)
int launch_bwd_dq(const BwdArgs& a, int head_dim, void* stream);
// fp32 only: the dQ kernel over the dQ schedule (writes dq; reads the D and
// lse2 of launch_bwd_pre)
int launch_bwd_dq_f32(const BwdArgs& a, int head_dim, void* stream);
int launch_fill(const FillArgs& a, void* stream);
// Size of the fixed device scratch used by swa_backward_noalloc, and the
// device address of the copy of it on the device of `stream` (null: the
// current device); looked up once per device (swa_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = SWA_NOALLOC_SCRATCH_BYTES;
int noalloc_scratch(void* stream, void** ptr, int* device);
const char* hip_error_string(int err);
int hip_memcpy_h2d_async(void* dst, const void* src, size_t bytes, void* stream);
int hip_pinned_alloc(void** p, size_t bytes);
int hip_pinned_free(void* p);
int hip_event_create(void** ev);
int hip_event_record(void* ev, void* stream);
int hip_event_sync(void* ev);
int hip_event_create_timed(void** ev);
int hip_event_elapsed_ms(float* ms, void* start, void* stop);
int hip_event_destroy(void* ev);
// compute units of the device of `stream` (null: the current device), cached per device
int hip_cu_count(void* stream, int* n);
// device of `stream` (null: the current device)
int hip_stream_device(void* stream, int* dev);
// device memory of `device` (allocated with that device current) and a
// synchronous host-to-device copy into it
int hip_device_alloc(int device, void** p, size_t bytes);
int hip_device_free(int device, void* p);  // waits for the device to be idle first
int hip_memcpy_h2d_sync(int device, void* dst, const void* src, size_t bytes);

}  // namespace swa
