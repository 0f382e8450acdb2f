// Helpers of the software-pipelined bf16 backward kernels (dK/dV and dQ):
// compile-time loops over pipeline slots and the transposing LDS operand
// reads.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "swa_common.hpp"

namespace swa {

#ifndef SWA_BWD_AHEAD
#define SWA_BWD_AHEAD 5
#endif
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Operands of the transposing reads (two 64-bit reads -> one 8 x bf16 operand)
__device__ inline bf16x8 tr_pair(const char* p0, const char* p1) {
  const shortx4 x = lds_read_tr16(p0);
  const shortx4 y = lds_read_tr16(p1);
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Lane offsets of the transposing operand reads of a swizzled [rows, RB]
// tile (accumulator row order, see tr_operand): rows 4h + l%16/4 and 8 more,
// head-dim block db.
template <int RB>
__device__ inline void tr_offsets(int lane, int db, int& o0, int& o1) {
  const int s16 = lane & 15, h = lane >> 5;
  const int col2 = 2 * (32 * db + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3));
  o0 = tile_off<RB>(4 * h + (s16 >> 2), col2);
  o1 = tile_off<RB>(4 * h + (s16 >> 2) + 8, col2);
}

}  // namespace swa
