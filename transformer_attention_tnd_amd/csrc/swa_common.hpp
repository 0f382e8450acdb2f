// Device-side helpers shared by the gfx950 attention kernels.
//
// Matrix-core fragments.  Every contraction uses a 32x32 output block:
//   bf16: v_mfma_f32_32x32x16_bf16  (each lane supplies 8 bf16 per operand)
//   fp32: v_mfma_f32_32x32x2_f32    (each lane supplies 1 float per operand)
// Operand A[i][k]: lane l supplies row i = l % 32 and the KPL consecutive
// contraction slots k = KSTEP*t + KPL*(l / 32) + e of step t.  Operand B[k][j]
// likewise with column j = l % 32.  The accumulator C (16 floats per lane)
// holds column j = l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
//
// A C fragment can feed the next contraction straight from registers when its
// rows become the contraction index: step t takes accumulator registers
// [KPL*t, KPL*t + KPL), i.e. contraction slot p corresponds to C row rho(p).
// The other operand of that contraction is then staged in LDS with its rows
// at position slot_of_row(row) = rho^-1(row), so that each lane still reads
// KPL consecutive elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_internal.hpp"

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef bf16x8 op_t;
  __device__ static inline floatx16 mma(op_t a, op_t b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  // accumulator registers [8t, 8t+8) rounded to bf16 (round to nearest even)
  __device__ static inline op_t pack(const floatx16& c, int t) {
    op_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = static_cast<bf16>(c[8 * t + e]);
    return r;
  }
};

template <>
struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float op_t;
  __device__ static inline floatx16 mma(op_t a, op_t b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const float* p) { return *p; }
  __device__ static inline op_t pack(const floatx16& c, int t) { return c[t]; }
};

// Row (within a 32-row block) of accumulator register r for lane half h.
__device__ __host__ constexpr inline int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Position in a transposed LDS row of the element whose C row is `row`.
template <typename T>
__device__ __host__ constexpr inline int slot_of_row(int row) {
  // bf16: rho swaps bits 2 and 3;  fp32: row = 8A + 4h + b  ->  8A + 2b + h
  return sizeof(T) == 2 ? ((row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1))
                        : ((row & ~31) | (((row >> 3) & 3) << 3) | ((row & 3) << 1) |
                           ((row >> 2) & 1));
}

// Inverse of slot_of_row: the C row whose value sits at contraction slot p.
template <typename T>
__device__ __host__ constexpr inline int row_of_slot(int p) {
  return sizeof(T) == 2 ? slot_of_row<T>(p)
                        : ((p & ~31) | (((p >> 3) & 3) << 3) | ((p & 1) << 2) | ((p >> 1) & 3));
}

// XOR swizzle of transposed LDS tiles (rows = head-dim index d, 64 positions
// per row): keeps aligned groups of 8 positions contiguous while spreading
// the transposing writes of consecutive 8-wide d chunks over distinct banks.
__device__ inline int swz(int d, int pos) { return pos ^ (((d >> 3) & 7) << 3); }

// 16-byte vector of elements.
struct alignas(16) Vec16 {
  uint32_t w[4];
};

template <typename T>
__device__ inline Vec16 load16(const T* p) {
  return *reinterpret_cast<const Vec16*>(p);
}

__device__ inline Vec16 zero16() {
  Vec16 v;
  v.w[0] = v.w[1] = v.w[2] = v.w[3] = 0u;
  return v;
}

template <typename T>
__device__ inline T vec_elem(const Vec16& v, int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = v.w[e >> 1];
    const uint16_t bits = (e & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xffff);
    return __builtin_bit_cast(bf16, bits);
  } else {
    return __builtin_bit_cast(float, v.w[e]);
  }
}

template <typename T>
__device__ inline float to_f32(T x) {
  return static_cast<float>(x);
}

// Workgroup index -> logical work index so that the workgroups of one XCD
// (dispatched round-robin, wg % 8) take a contiguous range of logical work.
__device__ inline int xcd_remap(int wg, int nwg) {
  const int x = wg & 7, idx = wg >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  return x * q + (x < r ? x : r) + idx;
}

__device__ inline bool allowed(int i, int j, int sq, int skv, int mode, int pre, int next) {
  if (i >= sq || j >= skv) return false;
  if (mode == 0) return true;
  const int d = j - i;
  return d >= -pre && d <= next;
}

}  // namespace swa
