// Helpers of the software-pipelined bf16 backward kernels (dK/dV and dQ):
// compile-time loops over pipeline slots and the transposing LDS operand
// reads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
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

// ---- work units of the persistent kernels
//
// A workgroup runs the units work[0 .. n) of its work list (codes
// item | head << 16).  The 16 words of a unit's item are held one per lane
// (lanes 0..15 of a register) from the time they are loaded until they are
// read out with readlane, so that the item of a later unit can be fetched
// while the current unit runs, with no scalar load outstanding in its loops.

static_assert(offsetof(Item, block) == 16 && offsetof(Item, tiles) == 24 &&
                  offsetof(Item, full) == 32 && offsetof(Item, band) == 40 &&
                  offsetof(Item, drop_base) == 48,
              "item words read by unit_info");

// Fields of a unit, uniform across the workgroup.
struct UnitInfo {
  int q_base, kv_base, sq, skv, block, tiles0, full0, pre, next, head;
  int64_t drop_base;
};

// Load of work[i] by every lane from a vector register address (a vector
// memory load, counted with the other vector-memory operations).
__device__ inline int32_t load_code(const int32_t* work, int i) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return work[i + z];
}

// A unit held one word per lane: lanes 0..15 the words of its item, lane 16
// its code (lanes 17..63: zero).
__device__ inline uint32_t load_unit(const Item* items, int32_t code, int lane) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(items + (code & 0xffff));
  return lane < 16 ? p[lane] : (lane == 16 ? (uint32_t)code : 0u);
}

// The fields of a unit held by load_unit.  The register passes an empty asm
// first, so that the reads happen here and are not hoisted to where the
// fields would stay live, in scalar registers, across the caller's loops.
__device__ inline UnitInfo unit_info(uint32_t iv) {
  asm volatile("" : "+v"(iv));
  auto word = [&](int k) { return __builtin_amdgcn_readlane((int)iv, k); };
  UnitInfo u;
  u.q_base = word(0);
  u.kv_base = word(1);
  u.sq = word(2);
  u.skv = word(3);
  u.block = word(4);
  u.tiles0 = word(6);
  u.full0 = word(8);
  u.pre = word(10);
  u.next = word(11);
  u.drop_base = (int64_t)(uint32_t)word(12) | ((int64_t)word(13) << 32);
  u.head = word(16) >> 16;
  return u;
}

}  // namespace swa
