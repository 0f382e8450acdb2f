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

// Swizzled row-major LDS tiles.  Rows are stored back to back with no
// padding; the 16-byte chunk c of row r sits at chunk c ^ tile_swz<RB>(r).
// Rows of 256 bytes or more use s(r) = 4 (r mod 4) + (r / 4 mod 4): a
// permutation of 16 consecutive rows, so that 16 rows reading one logical
// chunk (a 128-bit operand read) land on 16 distinct bank groups, and one
// that puts the 4 rows of each half-wave of a transposing 64-bit read (two
// aligned 32-byte pairs per row, from two 16-lane groups) in 4 different
// aligned groups of 4 chunks, so the half-wave covers all 64 banks once.
// 128-byte rows (8 chunks) use a 3-bit permutation.
template <int RB>
__device__ __host__ constexpr inline int tile_swz(int r) {
  return RB >= 256 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 3) << 1) | ((r >> 2) & 1));
}
template <int RB>
__device__ __host__ constexpr inline int tile_off(int r, int byte) {
  return r * RB + ((((byte >> 4) ^ tile_swz<RB>(r)) << 4) | (byte & 15));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, byte range nbytes) for the bounds-checked
// direct global->LDS loads; reads past nbytes return zeros.
__device__ inline u32x4 buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r = {(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nbytes, 0x00020000u};
  r.x = __builtin_amdgcn_readfirstlane(r.x);
  r.y = __builtin_amdgcn_readfirstlane(r.y);
  r.z = __builtin_amdgcn_readfirstlane(r.z);
  r.w = __builtin_amdgcn_readfirstlane(r.w);
  return r;
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const lds_void*)(p));
}

// The copies below set m0 (the LDS destination of a buffer load into LDS)
// themselves and list it as clobbered.  The compiler reserves m0 and sets it
// right before each of its own instructions that read it, so the clobber
// entry only documents the write; its warning about a reserved register in
// a clobber list is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// 16 bytes per lane from rsrc + voff into LDS at lds_base + 16 * lane.  The
// copy is issued as inline assembly so that the compiler does not treat it
// as an LDS store (it would otherwise wait for it before every later LDS
// read, even of other buffers); the caller waits with wait_vmem() and
// synchronises before the destination is read.
__device__ inline void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// dma16 with an extra scalar byte offset added to the source address.
__device__ inline void dma16_so(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// 4 bytes per lane from rsrc + voff into LDS at lds_base + 4 * lane (the
// same asynchronous global->LDS copy, one dword per lane).
__device__ inline void dma4(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// Copy rows [0, ROWS) of a row-major [rows, ld] slice starting at `base`
// into a swizzled LDS tile (no registers involved).  Rows >= nvalid read as
// zero.  All NT threads of the workgroup take part.
template <typename T, int D, int ROWS, int NT = 256>
__device__ inline void tile_load_lds(const T* base, int64_t ld, int nvalid, char* tile, int tid) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int SLOTS = ROWS * CPR;
  static_assert(SLOTS % NT == 0, "tile load mapping");
  const int64_t row_bytes = ld * (int64_t)sizeof(T);
  nvalid = nvalid < ROWS ? nvalid : ROWS;
  const uint32_t nrec = nvalid > 0 ? (uint32_t)((nvalid - 1) * row_bytes + RB) : 0u;
  const u32x4 rsrc = buffer_rsrc(base, nrec);
  const uint32_t tbase = lds_addr(tile);
#pragma unroll
  for (int p = 0; p < SLOTS / NT; ++p) {
    const int sl = p * NT + tid;
    const int row = sl / CPR, pc = sl % CPR;
    const uint32_t voff = (uint32_t)(row * row_bytes) + (uint32_t)((pc ^ tile_swz<RB>(row)) << 4);
    const uint32_t dst = __builtin_amdgcn_readfirstlane(tbase + (p * NT + (tid & ~63)) * 16);
    dma16(rsrc, voff, dst);
  }
}

// The copy of tile_load_lds in its PARTS separate instructions, so that a
// software pipeline can issue them one at a time between its other work (a
// burst of them stalls the issuing waves while the address unit drains
// them).  Part p covers rows p * NT / CPR .. of the tile; with NT / CPR a
// multiple of 16 every part has the same swizzle, so the parts differ only by
// a row-stride offset.
template <typename T, int D, int ROWS, int NT = 256>
struct TileDma {
  static constexpr int RB = D * (int)sizeof(T);
  static constexpr int CPR = RB / 16;
  static constexpr int PARTS = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0 && (NT / CPR) % 16 == 0, "tile load mapping");
  u32x4 rsrc;
  uint32_t voff, vstep, dst;
  __device__ void init(const T* base, int64_t ld, int nvalid, char* tile, int tid) {
    const int64_t row_bytes = ld * (int64_t)sizeof(T);
    nvalid = nvalid < ROWS ? nvalid : ROWS;
    rsrc = buffer_rsrc(base, nvalid > 0 ? (uint32_t)((nvalid - 1) * row_bytes + RB) : 0u);
    const int row = tid / CPR, pc = tid % CPR;
    voff = (uint32_t)(row * row_bytes) + (uint32_t)((pc ^ tile_swz<RB>(row)) << 4);
    vstep = (uint32_t)((NT / CPR) * row_bytes);
    dst = __builtin_amdgcn_readfirstlane(lds_addr(tile) + (tid & ~63) * 16);
  }
  template <int P>
  __device__ void issue() const {
    static_assert(P < PARTS, "part");
    dma16(rsrc, voff + P * vstep, dst + P * NT * 16);
  }
};

// Contiguous copy of `bytes` (a multiple of 16, at most 1024) into LDS by the
// first bytes/16 lanes of wave 0; bytes past `valid_bytes` read as zero.
__device__ inline void span_load_lds(const void* base, uint32_t valid_bytes, int bytes, char* dst,
                                     int tid) {
  if (tid < bytes / 16) {
    const u32x4 rsrc = buffer_rsrc(base, valid_bytes);
    dma16(rsrc, tid * 16, __builtin_amdgcn_readfirstlane(lds_addr(dst)));
  }
}

// Wait for this wave's outstanding vector-memory operations (vmcnt = 0).
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt immediate that waits until at most n (< 64) vector-memory
// operations are outstanding (vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima).
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

// Transposing 64-bit LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane j receives element (j & 3) of the 4-element chunks addressed by
// lanes (j >> 2), 4 + (j >> 2), 8 + (j >> 2), 12 + (j >> 2).
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ inline shortx4 lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

// bf16 operand (8 values) of lane l read from a swizzled row-major [rows, D]
// bf16 tile at column 32*db + (l & 31).  Element e (contraction slot
// 8*(l>>5) + e of the step starting at row0) is the tile row
//   kRho:  row0 + 8*(e>>2) + 4*(l>>5) + (e&3)   (accumulator row order)
//   else:  row0 + 8*(l>>5) + e                  (natural order)
template <int RB, bool kRho>
__device__ inline bf16x8 tr_operand(const char* tile, int row0, int db, int lane) {
  const int s = lane & 15, h = lane >> 5;
  const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int r = row0 + (kRho ? 4 : 8) * h + (s >> 2);
  const int r2 = r + (kRho ? 8 : 4);
  const shortx4 lo = lds_read_tr16(tile + tile_off<RB>(r, 2 * col));
  const shortx4 hi = lds_read_tr16(tile + tile_off<RB>(r2, 2 * col));
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Scheduling hints: ask the machine scheduler to interleave LDS reads with
// matrix instructions so that operands are fetched `ahead` instructions
// before their use (masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU).
template <int NMFMA, int READS_PER, int AHEAD>
__device__ inline void interleave_lds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, READS_PER * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + AHEAD < NMFMA) __builtin_amdgcn_sched_group_barrier(0x100, READS_PER, 0);
  }
}

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

// Store a wave's 32 rows of 32 NDB values held in transposed accumulators
// (lane l: row l % 32, value 32 db + 8 g + 4 (l / 32) + e in acc[db][4 g + e]),
// each value times mul and rounded to bf16, as whole rows.  Stored directly,
// a lane would write half of its row in 8-byte pieces and every store
// instruction would scatter over 64 rows, ld elements apart; here the rows go
// through the wave's own LDS slice st (32 swizzled rows of 64 NDB bytes,
// which no other wave may touch meanwhile) and each store instruction
// writes 16 bytes per lane, 64 / (4 NDB) complete rows.  Rows r >= nrows of
// dst are not written.
template <int NDB>
__device__ __attribute__((always_inline)) inline void store_rows_via_lds(const floatx16 (&acc)[NDB], float mul,
                                                                          char* st, bf16* dst, int64_t ld,
                                                                          int nrows) {
  constexpr int RB = 64 * NDB;  // row bytes
  // lane indices formed here (an empty asm keeps the compiler from sharing
  // these offsets with values computed before the caller's tile loop, which
  // would keep them live, in registers, across it)
  int ln = threadIdx.x;
  asm volatile("" : "+v"(ln));
  ln &= 63;
  const int c = ln & 31, h = ln >> 5;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = static_cast<bf16>(acc[db][4 * g + e] * mul);
      *reinterpret_cast<bf16x4*>(st + tile_off<RB>(c, 2 * (32 * db + 8 * g + 4 * h))) = v4;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads what its other lanes wrote
  constexpr int CPR = RB / 16, RPI = 64 / CPR;           // 16-byte chunks per row, rows per instruction
  constexpr int NI = 32 / RPI;                           // store instructions
  const int ch = ln % CPR, rr = ln / CPR;
  // the rows of a batch are all read before its stores: read inside each
  // row's store condition, each read would be waited for on its own
  constexpr int NB = NI >= 4 ? 4 : NI;  // rows per batch (registers permitting)
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NB) {
    u32x4 val[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      val[i] = *reinterpret_cast<const u32x4*>(st + tile_off<RB>(RPI * (i0 + i) + rr, 16 * ch));
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" : "+v"(val[i]));
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = RPI * (i0 + i) + rr;
      if (r < nrows) *reinterpret_cast<u32x4*>(dst + (int64_t)r * ld + 8 * ch) = val[i];
    }
  }
  asm volatile("" ::: "memory");  // the reads stay ahead of any later write to st
}

// Element mask: inside the sequence and, unless mode is 0, inside the band
// -pre <= j - i <= next (the item's band: sparse modes 2, 3 and 4 all reach the
// kernels in this form).
__device__ inline bool allowed(int i, int j, int sq, int skv, int mode, int pre, int next) {
  if (i >= sq || j >= skv) return false;
  if (mode == 0) return true;
  const int d = j - i;
  return d >= -pre && d <= next;
}

// A lane's allowed element offsets within one tile of n elements, as
// [lo, lo + w]: one subtract and one unsigned compare per element, all on the
// vector ALU (no scalar combine of two compare masks).  An empty range is
// lo = n, w = 0, which no offset in [0, n) passes.
struct LaneRange {
  int lo;
  unsigned w;
};
__device__ inline LaneRange lane_range(int lo, int hi, int n) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > n - 1 ? n - 1 : hi;
  LaneRange r;
  r.lo = hi < lo ? n : lo;
  r.w = hi < lo ? 0u : (unsigned)(hi - lo);
  asm volatile("" : "+v"(r.lo), "+v"(r.w));  // keep the per-lane form
  return r;
}
__device__ inline bool in_range(int rel, const LaneRange& r) {
  return (unsigned)(rel - r.lo) <= r.w;
}

}  // namespace swa
