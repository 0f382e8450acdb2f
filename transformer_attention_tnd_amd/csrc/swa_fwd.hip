// Forward kernel: online-softmax attention over the visited key tiles of one
// block of 256 query rows of one (sequence, head).
//
// Math (FlashAttentionVarLenScore API doc, "计算公式"; PyPTO-Gym
// FlashAttentionScoreGrad article, "前向公式"): out = softmax(mask(scale Q K^T)) V,
// with softmax_max / softmax_sum saved per row.  The blockwise (online)
// softmax keeps a running max and running sum per row, so the full score
// matrix never exists.
//
// Workgroup: 8 wavefronts in two groups of 4; group g owns rows
// [128 g, 128 g + 128) of the block, 32 rows per wave.  Each wave keeps its Q
// rows in registers and computes the transposed score block S^T = K Q^T
// (keys as rows, its 32 queries as columns), so that a lane owns one query
// row: row max and row sum are in-lane reductions plus one swap of lane
// halves.  The probabilities are rounded to the input type and fed from
// registers as the B operand of O^T += V^T P^T.
//
// Ping-pong: per key tile t a wave runs a matrix phase M(t) = {P(t-1) V(t-1),
// S(t) = K(t) Q^T} and a vector phase V(t) = softmax of S(t).  The two groups
// are offset by half a tile and separated by workgroup barriers:
//     half A:  group 0 runs M(t)   while group 1 runs V(t-1)
//     half B:  group 0 runs V(t)   while group 1 runs M(t)
// Each SIMD holds one wave of each group, so its matrix core always has one
// wave feeding it while the other wave's softmax runs on the vector ALUs.
//
// Tiles: the bf16 kernels without dropout walk 128-key tiles (two of the
// scheduler's 64-key tiles per step, which halves the barriers, rescale
// checks and lane swaps per key); the dropout and fp32 kernels walk 64-key
// tiles.
//
// Data movement: K and V tiles go from HBM straight into swizzled row-major
// LDS tiles (buffer loads with the LDS destination, rows past the sequence
// read as zero).  In the bf16 kernels without dropout the copies go out part
// by part from the matrix phases, into two buffers each at D = 128 (four at
// D = 64); otherwise they rotate through three buffers (two when three do
// not fit).  V^T operands come from the row-major V tile through
// transposing LDS reads.  The matrix phase (bf16) is one software pipeline of
// its products with the LDS operands read a few products ahead; it runs at
// raised wave priority.  At the end (bf16) each wave stages its 32 output
// rows in LDS and stores them as whole rows.
//
// Dropout (a kDrop instantiation): the keep bits of a lane's row for the
// tile are read as three 32-bit words in the matrix phase that forms the
// tile's scores and applied in its softmax, after the row sum.
//
// Rescaling: the exponent reference of a row is only moved when the running
// max exceeds it by more than 2^8 (in exp2 units); exp values then stay below
// 256, and the true max is tracked separately for softmax_max, with
// softmax_sum converted to it at the end.  The result is the same softmax.

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "swa_common.hpp"

namespace swa {

#ifndef SWA_FWD_AHEAD
#define SWA_FWD_AHEAD 3
#endif
template <typename F, int... I>
__device__ inline void fwd_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  fwd_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Maximum / sum of a value over the lane pair (l, l ^ 32): one lane-half
// swap in registers (v_permlane32_swap), no LDS round trip.
__device__ inline float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T, int D, bool kPos, bool kDrop>
__global__ __launch_bounds__(512, 1) void swa_fwd_kernel(FwdArgs a) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  // bf16 walks 128-key tiles (two of the scheduler's 64-key tiles per step:
  // half the barriers, rescale checks and lane swaps per key); fp32 walks
  // the scheduler's tiles
  constexpr bool kWide = sizeof(T) == 2;
  constexpr int HALF = FWD_HALF, BN = kWide ? 2 * FWD_BN : FWD_BN, NT = 512;
  constexpr int SUB = BN / FWD_BN;  // scheduler tiles per kernel tile
  constexpr int RB = D * (int)sizeof(T);  // tile row bytes
  constexpr int TB = BN * RB;             // tile bytes
  constexpr int NDB = D / 32;             // 32-wide head-dim blocks
  constexpr int NJB = BN / 32;            // 32-key blocks per tile
  constexpr int QSTEPS = D / KSTEP;       // contraction steps over d
  constexpr int PSTEPS = 32 / KSTEP;      // contraction steps per 32 keys
  constexpr float kRescale = 8.f;         // exp2-domain slack before moving the reference
  static_assert(HALF == 128 && FWD_BN == 64, "two groups of 4 waves x 32 rows; 64-key scheduler tiles");

  // K and V tiles rotate through NBUF buffers each: four for the bf16
  // kernels without dropout, whose copies are issued from the matrix phases
  // (the copy of a tile then has two steps to land), else three when they
  // fit (one step), else two
  constexpr bool kSpreadable = sizeof(T) == 2;
  constexpr int NBUF = kSpreadable && 8 * TB <= 160 * 1024   ? 4
                      : kSpreadable && 6 * TB <= 160 * 1024 ? 3
                      : 6 * TB <= 160 * 1024 && !kWide      ? 3
                                                            : 2;
  __shared__ __attribute__((aligned(1024))) char lds[2 * NBUF * TB];  // K[NBUF] V[NBUF]
  char* const kbuf0 = lds;
  char* const vbuf0 = lds + NBUF * TB;
  // bf16 dropout: the keep words of a tile for every row of the block (KW
  // words a row: the 128 keys of the tile span 5 words at any bit offset),
  // two tiles in turn
  constexpr bool kDropLds = kDrop && sizeof(T) == 2;
  constexpr int KW = 6;
  constexpr int KEEP_TILE = 2 * HALF * KW;  // words of one tile
  static_assert(!kDropLds || (BN == 128 && 32 * KW == 3 * 64), "three 64-lane copies per wave");
  __shared__ __attribute__((aligned(16))) uint32_t keep_lds[kDropLds ? 2 * KEEP_TILE : 1];

  const int64_t ld = (int64_t)a.num_heads * D;       // q / out row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v row stride
  // Persistent: this workgroup runs the units work[0 .. n_units) (an item of
  // 2 x HALF query rows and a head each, from the host's work list).
  const int32_t* work = a.work + a.work_off[blockIdx.x];
  const int n_units = a.work_off[blockIdx.x + 1] - a.work_off[blockIdx.x];
  if (n_units <= 0) return;
  // the bf16 kernels without dropout load a unit's Q rows and first tiles
  // before the previous unit's epilogue, which then stages its rows in the
  // last two V buffers (the first tiles take the others)
  constexpr bool kOverlap = sizeof(T) == 2;
  // a kernel tile is visited if one of its scheduler tiles is, and mask-free
  // only if all of them are (keys of a visited kernel tile that the schedule
  // skips are outside the band: the mask removes them)
  auto vis = [](int32_t r, int& l, int& u) {
    const int l0 = r & 0xffff, u0 = (r >> 16) & 0xffff;
    l = l0 > u0 ? 1 : l0 / SUB;
    u = l0 > u0 ? 0 : u0 / SUB;
  };
  // the loop range of a unit: the union of its two halves' visited tiles
  auto loop_range = [&](const Item& u, int& l, int& h) {
    int lo0, hi0, lo1, hi1;
    vis(u.tiles[0], lo0, hi0);
    vis(u.tiles[1], lo1, hi1);
    if (lo0 > hi0) {
      l = lo1;
      h = hi1;
    } else if (lo1 > hi1) {
      l = lo0;
      h = hi0;
    } else {
      l = lo0 < lo1 ? lo0 : lo1;
      h = hi0 > hi1 ? hi0 : hi1;
    }
  };
  // Q fragments: B operand of S^T = K Q^T, lane (column qrow) holds
  // Q[qrow][KSTEP*t + KPL*h + e].
  op_t qf[QSTEPS];
  // A unit's Q rows (into qf) and the copies of its first key / value tiles:
  // K(lo .. lo + NBUF - 2) and V(lo .. lo + NBUF - 3) into buffers 0, 1, ...
  auto unit_prologue = [&](const Item& u, int hd) {
    // lane indices formed here (the empty asm keeps them from being computed
    // once before the unit loop and held in registers across it)
    int t_ = threadIdx.x;
    asm volatile("" : "+v"(t_));
    const int tid = t_, lane = tid & 63, w = tid >> 6, g = w >> 2, h = lane >> 5, c = lane & 31;
    (void)lane;
    const int kh = hd / (a.num_heads / a.num_kv_heads);
    const int qr = u.block * 2 * HALF + HALF * g + 32 * (w & 3) + c;
    const bool ok = qr < u.sq;
    const T* qp = static_cast<const T*>(a.q) + ((int64_t)u.q_base + (ok ? qr : 0)) * ld + hd * D;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      qf[t] = M::load(qp + KSTEP * t + KPL * h);
      if (!ok) qf[t] = op_t{};
    }
    int ul, uh;
    loop_range(u, ul, uh);
    if (ul <= uh) {
      const T* kgu = static_cast<const T*>(a.k) + (int64_t)u.kv_base * ldkv + kh * D;
      const T* vgu = static_cast<const T*>(a.v) + (int64_t)u.kv_base * ldkv + kh * D;
      for (int j = 0; j <= NBUF - 2; ++j)
        if (ul + j <= uh)
          tile_load_lds<T, D, BN, NT>(kgu + (int64_t)(ul + j) * BN * ldkv, ldkv,
                                      u.skv - (ul + j) * BN, kbuf0 + j * TB, tid);
      for (int j = 0; j <= NBUF - 3; ++j)
        if (ul + j <= uh)
          tile_load_lds<T, D, BN, NT>(vgu + (int64_t)(ul + j) * BN * ldkv, ldkv,
                                      u.skv - (ul + j) * BN, vbuf0 + j * TB, tid);
    }
  };
  // the Q row loads are complete (the caller waited): an empty use of each
  // register tells the compiler's wait tracking, so that it does not count
  // them as outstanding in the loop (where a wait for them would also wait
  // for the tile copies in flight)
  auto settle_q = [&]() {
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) asm volatile("" : : "v"(qf[t]));
  };
  // Units' codes and items pass through LDS (bf16 with a positive scale; the
  // other kernels, short of registers, load them where needed): slot u & 1 holds the item of
  // unit u (words 0-15) and the codes of units u .. u + 3 (words 16-19, zero
  // past the list).  During unit u, lanes 0-3 of wave 0 copy those of unit
  // u + 1 into the other slot (copies waited for with the tile copies), so
  // that neither a unit's start nor its switch waits for a load.
  constexpr bool kSlots = sizeof(T) == 2 && kPos;
  __shared__ __attribute__((aligned(16))) int32_t unit_lds[2][20];
  auto fetch_unit = [&](int u, int32_t code) {  // unit u's item and codes into slot u & 1
    if (kSlots && threadIdx.x < 64) {
      span_load_lds(a.items + (code & 0xffff), (uint32_t)sizeof(Item), 64,
                    reinterpret_cast<char*>(unit_lds[u & 1]), threadIdx.x);
      span_load_lds(work + u, (uint32_t)(n_units - u) * 4u, 16,
                    reinterpret_cast<char*>(unit_lds[u & 1] + 16), threadIdx.x);
    }
  };
  auto slot_word = [&](int u, int i) { return __builtin_amdgcn_readfirstlane(unit_lds[u & 1][i]); };
  auto slot_item = [&](int u) {
    Item r;
    int32_t* d = reinterpret_cast<int32_t*>(&r);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = slot_word(u, i);
    return r;
  };
  {
    const int32_t code0 = work[0];
    fetch_unit(0, code0);
    unit_prologue(a.items[code0 & 0xffff], code0 >> 16);
    wait_vmem();
    settle_q();
    __syncthreads();
  }

  for (int ku = 0; ku < n_units; ++ku) {
  // lane indices formed again per unit (the empty asm keeps the compiler from
  // hoisting values derived from them out of the unit loop, where they would
  // hold registers across it)
  int tid_u = threadIdx.x;
  asm volatile("" : "+v"(tid_u));
  const int tid = tid_u;
  const int lane = tid & 63, w = tid >> 6, g = w >> 2, h = lane >> 5, c = lane & 31;
  const int w_u = w, h_u = h, c_u = c;
  const int32_t code = kSlots ? slot_word(ku, 16) : work[ku];
  const int head = code >> 16;
  const Item it = kSlots ? slot_item(ku) : a.items[code & 0xffff];
  if (kSlots && ku + 1 < n_units) fetch_unit(ku + 1, slot_word(ku, 17));
  const int kvh = head / (a.num_heads / a.num_kv_heads);  // grouped heads share K / V
  const T* kg = static_cast<const T*>(a.k) + (int64_t)it.kv_base * ldkv + kvh * D;
  const T* vg = static_cast<const T*>(a.v) + (int64_t)it.kv_base * ldkv + kvh * D;
  const int qrow = it.block * 2 * HALF + HALF * g + 32 * (w & 3) + c;  // sequence-local
  // this group's tile range, and the union over both groups (the loop range),
  // in kernel tiles
  auto full = [](int32_t r, int& l, int& u) {
    const int l0 = r & 0xffff, u0 = (r >> 16) & 0xffff;
    l = l0 > u0 ? 1 : (l0 + SUB - 1) / SUB;
    u = l0 > u0 ? 0 : (u0 + 1) / SUB - 1;
  };
  int mlo, mhi, mflo, mfhi;
  vis(g ? it.tiles[1] : it.tiles[0], mlo, mhi);
  full(g ? it.full[1] : it.full[0], mflo, mfhi);
  int lo, hi;
  loop_range(it, lo, hi);
  const float cs = kPos ? a.scale_log2 : 1.f;  // raw score -> exp2 units
  // Keys allowed for this lane's row: j in [j_min, j_max] (empty past the
  // end).  Formed where a masked tile needs it (the row index passes an
  // empty asm so the compiler does not keep the two bounds live, in
  // registers, across the whole loop).
  auto key_range = [&](int& j_min, int& j_max) {
    int q = qrow;
    asm volatile("" : "+v"(q));
    j_min = 0;
    j_max = it.skv - 1;
    if (a.mode != 0) {  // (the item's band is clamped to +-2^30 and q < 2^20: no overflow)
      const int lo32 = q - it.band[0], hi32 = q + it.band[1];
      j_min = lo32 < 0 ? 0 : (lo32 > it.skv ? it.skv : lo32);
      j_max = hi32 < j_max ? (hi32 < -1 ? -1 : hi32) : j_max;
    }
    if (q >= it.sq) j_max = -1;
  };

  // Dropout keep bits of this lane's row for the keys of a tile (bit k = key
  // BN t + k), funnel-shifted into the window in the tile's softmax.
  // fp32 (64-key tiles): three 32-bit words per lane; the words of tile t + 1
  // are loaded (into mwn) in the matrix phase of tile t and move into mw at
  // the start of the next matrix phase, so a load has a full step to land.
  uint32_t mw[3] = {0u, 0u, 0u}, mwn[3] = {0u, 0u, 0u};
  uint32_t msh = 0, mshn = 0;
  const int64_t drop_row = (kDrop && !kDropLds) ? it.drop_base + (int64_t)head * it.sq * it.skv +
                                                      (int64_t)(qrow < it.sq ? qrow : 0) * it.skv
                                                : 0;
  // bf16 (128-key tiles): the matrix phase of tile t copies the words of
  // tile t + 1 for the wave's 32 rows into keep_lds[(t + 1) % 2] (a row's
  // words are those of its clamped row: rows past the sequence attend
  // nothing), by three 4-byte global -> LDS copies per lane.  Bits are
  // addressed relative to X, the first bit of the wave's first (clamped) row:
  // row X + d skv starts in word (X % 32 + d skv) / 32 after word X / 32.
  // the wave's index and first row (wave-uniform: scalar registers)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int row0w = it.block * 2 * HALF + 32 * wu;
  auto keep_x = [&]() -> int64_t {
    return it.drop_base + (int64_t)head * it.sq * it.skv +
           (int64_t)(row0w < it.sq ? row0w : it.sq - 1) * it.skv;
  };
  auto load_keep = [&](int tile) {
    if constexpr (kDropLds) {
      int ln = threadIdx.x;
      asm volatile("" : "+v"(ln));
      ln &= 63;
      const int64_t X = keep_x();
      const int64_t wb = X >> 5;
      const int64_t left = (a.drop.n_words - wb) * 4;
      const u32x4 rs = buffer_rsrc(a.drop.words + wb, (uint32_t)(left < 0 ? 0 : (left > 0x7ffffffc ? 0x7ffffffc : left)));
      const uint32_t x5 = (uint32_t)(X & 31);
      const int rc0 = row0w < it.sq ? row0w : it.sq - 1;
      const uint32_t dst = lds_addr(keep_lds + (tile & 1) * KEEP_TILE + wu * 32 * KW);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int slot = 64 * i + ln, r = slot / KW, e = slot - KW * (slot / KW);
        const int rr = row0w + r;
        const uint32_t d = (uint32_t)((rr < it.sq ? rr : it.sq - 1) - rc0);
        const uint32_t word = ((x5 + d * (uint32_t)it.skv) >> 5) + 4u * (uint32_t)tile + (uint32_t)e;
        dma4(rs, 4u * word, __builtin_amdgcn_readfirstlane(dst + 256 * i));
      }
    }
  };
  auto load_mask = [&](int tile) {
    if constexpr (kDrop && !kDropLds) {
      const int64_t bit = drop_row + (int64_t)tile * BN;
      const int64_t w = bit >> 5;
      mshn = (uint32_t)(bit & 31);
#pragma unroll
      for (int e = 0; e < 3; ++e)
        mwn[e] = (qrow < it.sq && w + e < a.drop.n_words) ? a.drop.words[w + e] : 0u;
    }
  };

  auto load_k = [&](int tile, int b) {
    tile_load_lds<T, D, BN, NT>(kg + (int64_t)tile * BN * ldkv, ldkv, it.skv - tile * BN,
                                kbuf0 + b * TB, tid);
  };
  auto load_v = [&](int tile, int b) {
    tile_load_lds<T, D, BN, NT>(vg + (int64_t)tile * BN * ldkv, ldkv, it.skv - tile * BN,
                                vbuf0 + b * TB, tid);
  };

  floatx16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = floatx16{};
  float m_true = -INFINITY;  // running max of the raw (masked) scores
  float m_ref = -INFINITY;   // exponent reference, raw units
  float l_run = 0.f;         // running sum relative to m_ref (this lane's half)
  floatx16 s[NJB];           // scores of the current tile
  op_t pk[NJB][PSTEPS];      // probabilities of the previous tile, operand layout

  // S^T block jb: rows = keys 32*jb + c_row(r, h), column = this lane's query
  // (the two key blocks alternate so that consecutive MFMAs are independent)
  // (fp32 only; the lane indices are formed inside, behind an empty asm, so
  // that the compiler does not compute the many swizzled LDS offsets once
  // and hold them in registers across the tile loop)
  auto scores = [&](const char* kt) __attribute__((always_inline)) {
    int ln = threadIdx.x;
    asm volatile("" : "+v"(ln));
    const int c = ln & 31, h = (ln >> 5) & 1;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) s[jb] = floatx16{};
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const op_t ka = M::load(reinterpret_cast<const T*>(
            kt + tile_off<RB>(32 * jb + c, (KSTEP * t + KPL * h) * (int)sizeof(T))));
        s[jb] = M::mma(ka, qf[t], s[jb]);
      }
    }
  };
  // O^T[db] += V^T P^T with the probabilities of the previous tile (fp32
  // only; lane indices formed inside, as in scores)
  auto pv = [&](const char* vt) __attribute__((always_inline)) {
    int ln = threadIdx.x;
    asm volatile("" : "+v"(ln));
    const int c = ln & 31, h = (ln >> 5) & 1;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
      for (int t2 = 0; t2 < PSTEPS; ++t2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int row = 32 * jb + row_of_slot<T>(KSTEP * t2 + KPL * h);
          const op_t va =
              *reinterpret_cast<const T*>(vt + tile_off<RB>(row, (32 * db + c) * (int)sizeof(T)));
          o[db] = M::mma(va, pk[jb][t2], o[db]);
        }
      }
    }
  };
  // Softmax of the current tile: scores -> probabilities (packed), running stats.
  auto softmax = [&](auto mask_tag, int tile) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    if constexpr (!kPos) {  // non-positive scale: work on scaled scores (scale before masking)
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) s[jb] *= a.scale_log2;
    }
    if constexpr (kMask) {
      // key 32 jb + c_row(r, h) of the tile is allowed iff 32 jb + 8 (r / 4) + r % 4
      // lies in the lane's range (the 4 h of c_row moved into the bounds)
      int j_min, j_max;
      key_range(j_min, j_max);
      const LaneRange rg = lane_range(j_min - tile * BN - 4 * h, j_max - tile * BN - 4 * h, BN);
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = 32 * jb + 8 * (r >> 2) + (r & 3);
          s[jb][r] = in_range(rel, rg) ? s[jb][r] : -INFINITY;
        }
      }
    }
    // four independent partial maxima / sums keep the dependency chains short
    float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mp[r & 3] = fmaxf(mp[r & 3], s[jb][r]);
    }
    const float mx = pair_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
    m_true = fmaxf(m_true, mx);
    if (__ballot((m_true - m_ref) * cs > kRescale)) {
      const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_true) * cs);
      m_ref = m_true;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    const float moff = m_ref == -INFINITY ? 0.f : -m_ref * cs;
    // keep bits of this lane's keys: block jb, register r -> key 32 jb + c_row(r, h)
    uint32_t keep[NJB] = {};
    if constexpr (kDropLds) {
      // this lane's row: words from keep_lds, shift (X + d skv) % 32
      const uint32_t* kr = keep_lds + (tile & 1) * KEEP_TILE + (wu * 32 + c) * KW;
      const uint2 w01 = *reinterpret_cast<const uint2*>(kr);
      const uint2 w23 = *reinterpret_cast<const uint2*>(kr + 2);
      const uint32_t w4 = kr[4];
      const int rc0 = row0w < it.sq ? row0w : it.sq - 1;
      const uint32_t d = (uint32_t)((qrow < it.sq ? qrow : it.sq - 1) - rc0);
      const uint32_t sh = ((uint32_t)(keep_x() & 31) + d * (uint32_t)it.skv) & 31u;
      keep[0] = __builtin_amdgcn_alignbit(w01.y, w01.x, sh) >> (4 * h);
      keep[1] = __builtin_amdgcn_alignbit(w23.x, w01.y, sh) >> (4 * h);
      keep[2] = __builtin_amdgcn_alignbit(w23.y, w23.x, sh) >> (4 * h);
      keep[3] = __builtin_amdgcn_alignbit(w4, w23.y, sh) >> (4 * h);
    } else if constexpr (kDrop) {
      keep[0] = __builtin_amdgcn_alignbit(mw[1], mw[0], msh) >> (4 * h);
      keep[1] = __builtin_amdgcn_alignbit(mw[2], mw[1], msh) >> (4 * h);
    }
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[jb][r], cs, moff));
        ls[r & 3] += p;  // the row sum is that of the undropped softmax
        if constexpr (kDrop && !kDropLds) {
          // the signed one-bit field extract is 0 or all ones: a mask of p
          // (written as asm: the builtin is turned into an and, a compare and
          // a select, one instruction more); the factor 1 / keep_prob of the
          // kept terms is applied to the row at the end
          uint32_t m;
          asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(keep[jb]), "n"(8 * (r >> 2) + (r & 3)));
          s[jb][r] = __uint_as_float(__float_as_uint(p) & m);
        } else {
          s[jb][r] = p;
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < PSTEPS; ++t2) pk[jb][t2] = M::pack(s[jb], t2);
      if constexpr (kDropLds) {
        // The keep bits mask the rounded probabilities a pair at a time:
        // dword i of operand t2 holds registers r = 8 t2 + 2 i and r + 1,
        // whose bits are b = 8 (r / 4) + r % 4 and b + 1, i.e. b0 = 8 (i / 2)
        // + 2 (i % 2) and b0 + 1 for t2 = 0, and 16 more for t2 = 1.  With
        // bit b0 shifted to bit 15 of x and bit b0 + 1 to bit 15 of y (so
        // bits b0 + 16, b0 + 17 sit at bit 31), v_perm_b32's selectors 8 / 10
        // (9 / 11) copy the sign bit of byte 1 (byte 3) of x / y into a whole
        // byte: the two 16-bit halves of the mask, for t2 = 0 (t2 = 1).
        // The factor 1 / keep_prob of the kept terms is applied to the row
        // at the end.
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        u32x4_t d0 = __builtin_bit_cast(u32x4_t, pk[jb][0]);
        u32x4_t d1 = __builtin_bit_cast(u32x4_t, pk[jb][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b0 = 8 * (i >> 1) + 2 * (i & 1);
          const uint32_t x = keep[jb] << (15 - b0), y = keep[jb] << (14 - b0);
          d0[i] &= __builtin_amdgcn_perm(y, x, 0x0A0A0808u);
          d1[i] &= __builtin_amdgcn_perm(y, x, 0x0B0B0909u);
        }
        pk[jb][0] = __builtin_bit_cast(op_t, d0);
        pk[jb][1] = __builtin_bit_cast(op_t, d1);
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // bf16 matrix phase as one software pipeline over its products: first
  // O^T += V^T P^T of the previous tile (PVN products, the head-dim blocks
  // innermost so consecutive products use different accumulators), then
  // S^T = K Q^T (SN products, the two key blocks alternating).  Each LDS
  // operand is read AHEAD products before use into a small register ring;
  // scheduling fences keep the order.
  constexpr int PVN = NJB * PSTEPS * NDB, SN = QSTEPS * NJB;
  constexpr int AHEAD = SWA_FWD_AHEAD, RING = AHEAD + 1;
  // LDS offsets of the operand reads: ok_[t], the 128-bit read of key row c,
  // chunk 2t + h; otr[db], the transposing reads of the V tile, head-dim
  // block db.  Formed once per unit, except ok_ with dropout, whose extra
  // state leaves no room to hold all of them across the tile loop: there
  // each matrix phase forms ok_ again from a lane index behind an empty asm
  // (measured: holding otr and forming ok_ per phase is the fastest of the
  // four ways, with no register spilled; holding both spilled 3 registers,
  // holding ok_ alone 82).
  int ok_[QSTEPS];
  int otr[NDB][2];
  auto operand_offsets = [&](int ln, auto part) __attribute__((always_inline)) {
    // part: 1 the 128-bit read offsets, 2 the transposing ones, 3 both
    constexpr int P = decltype(part)::value;
    if constexpr (sizeof(T) == 2) {
      ln &= 63;
      const int cc = ln & 31, hh = ln >> 5;
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t)
        if constexpr ((P & 1) != 0) ok_[t] = tile_off<RB>(cc, (KSTEP * t + KPL * hh) * 2);
#pragma unroll
      for (int db = 0; db < NDB && (P & 2) != 0; ++db) {
        const int s16 = ln & 15;
        const int col2 = 2 * (32 * db + 16 * ((ln >> 4) & 1) + 4 * (s16 & 3));
        otr[db][0] = tile_off<RB>(4 * hh + (s16 >> 2), col2);
        otr[db][1] = tile_off<RB>(4 * hh + (s16 >> 2) + 8, col2);
      }
    }
  };
  // offsets formed per matrix phase (1: the 128-bit read offsets; with
  // dropout) and once per unit (the others)
  constexpr int kOffPerPhase = kDropLds ? 1 : 0;
  operand_offsets(lane, std::integral_constant<int, 3 - kOffPerPhase>{});
  // bf16 without dropout: each group copies one tile per step, part by part
  // from the slots of its matrix phase (a burst of copy instructions holds
  // the issuing waves while the address unit drains it): group 0 the K tile
  // NBUF - 1 steps ahead, group 1 the V tile NBUF - 2 steps ahead.
  // Past the range the copy reads nothing and writes zeros into the free
  // buffer, so every wave issues the same number of copies in every step.
  constexpr bool kSpread = kSpreadable;
  using Dma = TileDma<bf16, D, BN, 256>;  // (used by the bf16 instantiations only)
  constexpr int COPY_EVERY = 4;  // pipeline slots between copy instructions
  Dma cp;
  auto copy_burst = [&]() {
    static_for<Dma::PARTS>([&](auto pc) { cp.template issue<decltype(pc)::value>(); });
  };
  auto pipeline = [&](auto first_c, auto last_c, const char* kt, const char* vt) {
    constexpr int FIRST = decltype(first_c)::value, LAST = decltype(last_c)::value;
    static_assert(!kSpread || COPY_EVERY * (Dma::PARTS - 1) + 1 < LAST - FIRST + AHEAD,
                  "every copy has a slot");
    op_t ring[RING];
    if constexpr (kOffPerPhase != 0) {
      int ln = threadIdx.x;
      asm volatile("" : "+v"(ln));
      operand_offsets(ln, std::integral_constant<int, kOffPerPhase>{});
    }
    auto read = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (sizeof(T) != 2) {
        // fp32 runs the unpipelined phase
      } else if constexpr (i < PVN) {
        constexpr int jb = i / (PSTEPS * NDB), t2 = (i / NDB) % PSTEPS, db = i % NDB;
        constexpr int imm = (32 * jb + KSTEP * t2) * RB;
        typedef short shortx8 __attribute__((ext_vector_type(8)));
        const shortx4 x = lds_read_tr16(vt + otr[db][0] + imm);
        const shortx4 y = lds_read_tr16(vt + otr[db][1] + imm);
        const shortx8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        ring[i % RING] = __builtin_bit_cast(op_t, v);
      } else {
        constexpr int j = i - PVN, t = j / NJB, jb = j % NJB;
        ring[i % RING] = *reinterpret_cast<const op_t*>(kt + ok_[t] + 32 * jb * RB);
      }
    };
    auto mfma = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const op_t& x = ring[i % RING];
      if constexpr (i < PVN) {
        constexpr int jb = i / (PSTEPS * NDB), t2 = (i / NDB) % PSTEPS, db = i % NDB;
        o[db] = M::mma(x, pk[jb][t2], o[db]);
      } else {
        constexpr int j = i - PVN, t = j / NJB, jb = j % NJB;
        s[jb] = M::mma(x, qf[t], t == 0 ? floatx16{} : s[jb]);
      }
    };
    static_for<LAST - FIRST + AHEAD>([&](auto sc) {
      constexpr int sl = decltype(sc)::value;
      if constexpr (kSpread && sl % COPY_EVERY == 1 && sl / COPY_EVERY < Dma::PARTS)
        cp.template issue<sl / COPY_EVERY>();
      if constexpr (sl < LAST - FIRST) read(std::integral_constant<int, FIRST + sl>{});
      if constexpr (sl >= AHEAD) mfma(std::integral_constant<int, FIRST + sl - AHEAD>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // matrix phase M(t): P(t-1) V(t-1) and S(t), for the tiles of this group
  auto m_phase = [&](int t, int k) __attribute__((always_inline)) {
    const bool do_pv = t - 1 >= mlo && t - 1 <= mhi;
    const bool do_s = t >= mlo && t <= mhi;
    if constexpr (kDropLds) {  // the next tile's words, ahead of this step's tile copies
      if (t + 1 > mlo && t + 1 <= mhi) load_keep(t + 1);
    } else if constexpr (kDrop) {  // this tile's words in, the next tile's requested
#pragma unroll
      for (int e = 0; e < 3; ++e) mw[e] = mwn[e];
      msh = mshn;
      load_mask(t + 1);
    }
    const char* kt = kbuf0 + (k % NBUF) * TB;                 // K(t)
    const char* vt = vbuf0 + ((k + NBUF - 1) % NBUF) * TB;    // V(t-1)
    // the matrix phase takes issue priority over the other group's softmax
    // on the same SIMD (measured: about 2 % faster than equal priority)
    __builtin_amdgcn_s_setprio(3);
    if constexpr (sizeof(T) == 2) {
      using Z = std::integral_constant<int, 0>;
      using P = std::integral_constant<int, PVN>;
      using E = std::integral_constant<int, PVN + SN>;
      if (do_pv && do_s)
        pipeline(Z{}, E{}, kt, vt);
      else if (do_pv)
        pipeline(Z{}, P{}, kt, vt);
      else if (do_s)
        pipeline(P{}, E{}, kt, vt);
      else if constexpr (kSpread)
        copy_burst();
    } else {
      if (do_pv && do_s) {
        pv(vt);
        scores(kt);
      } else if (do_pv) {
        pv(vt);
      } else if (do_s) {
        scores(kt);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // vector phase V(t)
  auto v_phase = [&](int t) __attribute__((always_inline)) {
    if (t < mlo || t > mhi) return;
    if (t < mflo || t > mfhi)
      softmax(std::true_type{}, t);
    else
      softmax(std::false_type{}, t);
  };

  // copy instructions per thread for one K or V tile
  constexpr int NC = BN * (RB / 16) / NT;
  static_assert(2 * NC <= 15, "copy batch fits the wait immediate");
  static_assert(!kSpread || (NBUF - 2) * Dma::PARTS <= 15, "copies in flight fit the wait immediate");
  if (lo <= hi) {
    // (the Q rows and the first tiles were loaded by unit_prologue)
    if constexpr (kDropLds) {
      if (mlo <= mhi) load_keep(mlo);
      wait_vmem();
    } else if constexpr (kDrop) {
      load_mask(lo);
      wait_vmem();
    }
    const int nk = hi - lo + 2;
    for (int k = 0; k < nk; ++k) {
      const int t = lo + k;
      // copies: three buffers: K(t+2), V(t+1) (used two steps on);
      // two buffers: K(t+1), V(t) (used in the next step)
      const bool ck = NBUF == 3 ? t + 2 <= hi : t + 1 <= hi;
      const bool cv = NBUF == 3 ? t + 1 <= hi : t <= hi;
      if constexpr (kSpread) {
        // K(t + NBUF - 1) into the buffer of K(t - 1), V(t + NBUF - 2) into
        // that of V(t - 2): both last read in the previous step
        const int tt = g == 0 ? t + NBUF - 1 : t + NBUF - 2;
        const bf16* src = reinterpret_cast<const bf16*>(g == 0 ? kg : vg) + (int64_t)tt * BN * ldkv;
        char* dst = g == 0 ? kbuf0 + ((k + NBUF - 1) % NBUF) * TB : vbuf0 + ((k + NBUF - 2) % NBUF) * TB;
        cp.init(src, ldkv, tt <= hi ? it.skv - tt * BN : 0, dst, tid & 255);
      } else {
        if (ck) load_k(NBUF == 3 ? t + 2 : t + 1, (k + (NBUF == 3 ? 2 : 1)) % NBUF);
        if (cv) load_v(NBUF == 3 ? t + 1 : t, (k + (NBUF == 3 ? 1 : 0)) % NBUF);
      }
      // half A
      if (g == 0)
        m_phase(t, k);
      else
        v_phase(t - 1);
      __syncthreads();
      // half B
      if (g == 0)
        v_phase(t);
      else
        m_phase(t, k);
      // the tiles of the next step have landed (with three buffers, the
      // copies issued in this step may still be in flight)
      if constexpr (kSpread)  // the copies of the last NBUF - 2 steps (one tile per wave each) stay
        // in flight (with dropout only this step's, issued after the keep words)
        __builtin_amdgcn_s_waitcnt(0x0F70 | ((kDropLds && NBUF > 3 ? 1 : NBUF - 2) * Dma::PARTS));
      else if (NBUF == 2 || (!ck && !cv) || kDrop)  // dropout: the next tile's keep words too
        wait_vmem();
      else if (ck && cv)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NC));
      else
        __builtin_amdgcn_s_waitcnt(0x0F70 | NC);
      if constexpr (kDrop && !kDropLds) asm volatile("" : : "v"(mwn[0]), "v"(mwn[1]), "v"(mwn[2]), "v"(mshn));
      __syncthreads();
    }
    if constexpr (kSpread) {  // the last step's copies (into free buffers), of every wave
      wait_vmem();
      __syncthreads();
    }
  }

  // the next unit's Q rows and first tiles go out first (bf16 without
  // dropout) or after this unit's rows have left the K / V area; its slot
  // has landed (the tile loop ended with a wait and a barrier; a unit
  // without tiles waits here)
  const bool has_next = ku + 1 < n_units;
  if (kSlots && lo > hi) {
    wait_vmem();
    __syncthreads();
  }
  Item nit;
  int nhead = 0;
  if (has_next) {
    const int32_t ncode = kSlots ? slot_word(ku + 1, 16) : work[ku + 1];
    nhead = ncode >> 16;
    nit = kSlots ? slot_item(ku + 1) : a.items[ncode & 0xffff];
    if constexpr (kOverlap) unit_prologue(nit, nhead);
    // (measured: waiting for these loads before the epilogue's stores is
    // faster than letting the two overlap)
    if constexpr (kSlots) wait_vmem();
  }

  // epilogue: normalise, store out and the statistics of this lane's row.
  // (kSlots: its lane indices are formed again here; held from the unit's
  // start they may come back from scratch, and such reloads would wait
  // behind the next unit's row loads and tile copies issued above.)
  {
  int tid_e = threadIdx.x;
  if constexpr (kSlots) asm volatile("" : "+v"(tid_e));
  const int w = kSlots ? __builtin_amdgcn_readfirstlane(tid_e >> 6) : w_u;
  const int h = kSlots ? (tid_e & 63) >> 5 : h_u, c = kSlots ? tid_e & 31 : c_u;
  const int qrow = it.block * 2 * HALF + HALF * (w >> 2) + 32 * (w & 3) + c;  // sequence-local
  const float l_ref = pair_sum(l_run);
  // (dropout: times 1 / keep_prob, the factor of every kept term)
  const float inv = l_ref > 0.f ? (kDrop ? a.drop.rkp : 1.f) / l_ref : 0.f;
  const int64_t tok = (int64_t)it.q_base + qrow;
  if constexpr (sizeof(T) == 2) {
    // the wave's 32 rows as whole rows, through its own 32-row slice of the
    // K / V area (free once every wave has left the loop and the last
    // copies have landed): with kOverlap the last two V buffers
    static_assert(8 * 32 * RB <= 2 * NBUF * TB, "the staging slices fit in the K / V area");
    static_assert(!kOverlap || 8 * 32 * RB <= 2 * TB, "the staging slices fit in two V buffers");
    char* const stage = kOverlap ? vbuf0 + (NBUF - 2) * TB : lds;
    __syncthreads();
    const int row0 = it.block * 2 * HALF + 32 * w;  // sequence-local row of the wave's slice
    store_rows_via_lds<NDB>(o, inv, stage + w * 32 * RB,
                            static_cast<bf16*>(a.out) + ((int64_t)it.q_base + row0) * ld + head * D, ld,
                            it.sq - row0);
  } else if (qrow < it.sq) {
    T* op = static_cast<T*>(a.out) + tok * ld + head * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * db + 8 * gq + 4 * h;
        floatx4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * gq + e] * inv;
        *reinterpret_cast<floatx4*>(op + d0) = v4;
      }
    }
  }
  if (qrow < it.sq) {
    // statistics in natural units relative to the true max
    const bool empty = m_true == -INFINITY;
    const float smax = empty ? -INFINITY : m_true * cs * 0.69314718055994531f;
    const float ssum = empty ? 0.f : l_ref * __builtin_amdgcn_exp2f((m_ref - m_true) * cs);
    const floatx4 mv = {smax, smax, smax, smax};
    const floatx4 sv = {ssum, ssum, ssum, ssum};
    const int64_t so = (tok * a.num_heads + head) * 8 + 4 * h;
    *reinterpret_cast<floatx4*>(a.smax + so) = mv;
    *reinterpret_cast<floatx4*>(a.ssum + so) = sv;
  }
  }
  if (has_next) {
    if constexpr (!kOverlap) {
      __syncthreads();  // every wave's rows have left the K / V area
      unit_prologue(nit, nhead);
    }
    wait_vmem();
    settle_q();
    __syncthreads();
  }
  }  // units
}

template <typename T, int D, bool kDrop>
static int launch_fwd_t(const FwdArgs& a, void* stream) {
  const int64_t nwg = a.n_wg;  // persistent: one workgroup per compute unit
  if (a.scale_log2 > 0.f)
    hipLaunchKernelGGL((swa_fwd_kernel<T, D, true, kDrop>), dim3((unsigned)nwg), dim3(512), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_fwd_kernel<T, D, false, kDrop>), dim3((unsigned)nwg), dim3(512), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

template <bool kDrop>
static int launch_fwd_d(const FwdArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return head_dim == 128 ? launch_fwd_t<bf16, 128, kDrop>(a, stream)
                                         : launch_fwd_t<bf16, 64, kDrop>(a, stream);
  return head_dim == 128 ? launch_fwd_t<float, 128, kDrop>(a, stream)
                         : launch_fwd_t<float, 64, kDrop>(a, stream);
}

int launch_forward(const FwdArgs& a, int dtype, int head_dim, void* stream) {
  return a.drop.words ? launch_fwd_d<true>(a, dtype, head_dim, stream)
                      : launch_fwd_d<false>(a, dtype, head_dim, stream);
}

}  // namespace swa
