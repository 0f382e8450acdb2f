// Backward kernels.
//
// Math (PyPTO-Gym FlashAttentionScoreGrad article, "反向公式";
// aclnnFlashAttentionUnpaddingScoreGradV2 explainer, section 2.3):
//   P  = exp(scale Q K^T - softmax_max) / softmax_sum    (saved statistics)
//   D  = rowsum(dY * O)
//   dP = dY V^T,  dS = P * (dP - D)
//   dV = P^T dY,  dK = scale dS^T Q,  dQ = scale dS K
// in the explainer's stage order (section 8.3): recompute p, dp, ds, then the
// three products.
//
// swa_bwd_pre_kernel: D and the per-row log2-domain normaliser
//   lse2 = softmax_max * log2(e) + log2(softmax_sum), so that P = exp2(s*c - lse2)
//   with c = scale * log2(e); for fp32 it also zeroes the dq accumulator.
// bf16: swa_bwd_kv_kernel (dK, dV, in swa_bwd_kv.hip) and swa_bwd_dq_kernel
//   (dQ, in swa_bwd_dq.hip), the two-pass structure with no atomics.
// fp32: swa_bwd_kernel, one pass: one workgroup per (block of 128 keys,
//   head); each of its 4 waves owns 32 keys and keeps its dK, dV
//   accumulators in registers while it walks the query tiles of the band.
//   Scores are formed as S = Q K^T (queries as rows, the wave's keys as
//   columns), so P and dS come out of the accumulators in the operand layout
//   of dV^T += dY^T P and dK^T += Q^T dS.  Q and dY tiles go from HBM
//   straight into swizzled row-major LDS tiles (double-buffered, rows past
//   the sequence read as zero).  dS is written to LDS and each wave forms dQ
//   for one 32-wide head-dim block over all 128 keys, added to the fp32
//   accumulator with atomics (non-deterministic summation order, as the
//   explainer section 6.1 describes for the default backward);
//   swa_dq_finalize_kernel then writes dq = scale * dq_acc in the output type.
//   With grouped heads the workgroup of a key/value head walks the query
//   heads of its group in turn; with dropout the keep bits of each query tile
//   are staged in LDS next to lse2 and D.

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "swa_common.hpp"

namespace swa {

template <typename T, int D>
__global__ __launch_bounds__(256) void swa_bwd_pre_kernel(BwdPreArgs a) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int TPR = D / EPV;   // threads per row
  constexpr int RPB = 256 / TPR; // rows per workgroup
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int ch = threadIdx.x % TPR;
  if (row >= a.rows) return;  // whole row groups leave together
  const T* dy = static_cast<const T*>(a.dy) + row * D + ch * EPV;
  const T* o = static_cast<const T*>(a.out) + row * D + ch * EPV;
  const Vec16 vy = load16(dy), vo = load16(o);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc += to_f32(vec_elem<T>(vy, e)) * to_f32(vec_elem<T>(vo, e));
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (a.dq_acc) {
    float* z = a.dq_acc + row * D + ch * EPV;
#pragma unroll
    for (int e = 0; e < EPV; e += 4) *reinterpret_cast<floatx4*>(z + e) = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  if (ch == 0) {
    const int64_t tok = row / a.num_heads, head = row - tok * a.num_heads;
    const int64_t at = head * a.t_q + tok;  // head-major so that a tile's rows are contiguous
    a.drow[at] = acc;
    const float mx = a.smax[row * 8], sm = a.ssum[row * 8];
    a.lse2[at] = (sm > 0.f && mx > -INFINITY) ? mx * 1.4426950408889634f + log2f(sm) : INFINITY;
  }
}

template <typename T, int D, int BM, bool kDrop>
__global__ __launch_bounds__(256, 1) void swa_bwd_kernel(BwdArgs a) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int BN = BWD_BN;
  constexpr int ES = (int)sizeof(T);
  constexpr int RB = D * ES;              // Q / dY / K tile row bytes
  constexpr int QTB = BM * RB;            // Q or dY tile bytes
  constexpr int KTB = BN * RB;            // K block bytes
  constexpr int SRB = BN * ES;            // dS tile row bytes
  constexpr int STB = BM * SRB;           // dS tile bytes
  constexpr int NDB = D / 32;             // head-dim blocks
  constexpr int QB = BM / 32;             // 32-row query blocks per tile
  constexpr int DSTEPS = D / KSTEP;       // contraction steps over d
  constexpr int QSTEPS = 32 / KSTEP;      // contraction steps per 32 query rows
  constexpr int KSTEPS = BN / KSTEP;      // contraction steps over the 128 keys
  constexpr int WPD = 4 / NDB;            // waves sharing one head-dim block in dQ
  constexpr int TASKS = QB * NDB / 4;     // dQ output blocks per wave
  static_assert(BN == 128 && (BM == 64 || BM == 32), "4 waves x 32 keys; 32/64-row tiles");
  static_assert(NDB <= 4 && 4 % NDB == 0 && TASKS >= 1 && QB * NDB % 4 == 0, "dQ split");

  // bf16 reads the B operands of S and dP (K and V rows) from LDS; fp32
  // (one element per lane and step) keeps them in registers instead.
  constexpr bool kKVlds = sizeof(T) == 2;
  __shared__ __attribute__((aligned(1024))) char lds[4 * QTB + (kKVlds ? 2 : 1) * KTB + STB];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BM];
  __shared__ __attribute__((aligned(16))) float drow_s[2][BM];
  // dropout keep bits of the tile: [slot][key word kw / 32 of the block][row]
  __shared__ __attribute__((aligned(16))) uint32_t mask_s[kDrop ? 2 * 4 * BM : 1];
  char* const qbuf = lds;               // Q tiles [2]
  char* const ybuf = lds + 2 * QTB;     // dY tiles [2]
  char* const kblk = lds + 4 * QTB;     // K block (operand of S and of dQ)
  char* const vblk = kblk + KTB;        // V block (operand of dP)
  char* const sbuf = kKVlds ? vblk + KTB : vblk;  // dS tile

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kvh = L / a.n_items;  // the grid runs over key/value heads
  const Item it = a.items[L - kvh * a.n_items];
  const int N = a.num_heads;
  const int G = N / a.num_kv_heads;                  // query heads sharing this K / V
  const int64_t ld = (int64_t)N * D;                 // q / dy / dq row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v / dk / dv row stride
  const T* kg = static_cast<const T*>(a.k) + (int64_t)it.kv_base * ldkv + kvh * D;
  const T* vg = static_cast<const T*>(a.v) + (int64_t)it.kv_base * ldkv + kvh * D;
  // the query head being processed (the group's heads run one after another,
  // accumulating into the same dK / dV) and its tensors
  int head = kvh * G;
  const T* qg = nullptr;
  const T* dyg = nullptr;
  const float* lse_g = nullptr;
  const float* drow_g = nullptr;
  int64_t drop_head = 0;  // first dropout-mask bit of (sequence, query head)
  auto set_head = [&](int hq) {
    head = hq;
    drop_head = it.drop_base + (int64_t)hq * it.sq * it.skv;
    qg = static_cast<const T*>(a.q) + (int64_t)it.q_base * ld + hq * D;
    dyg = static_cast<const T*>(a.dy) + (int64_t)it.q_base * ld + hq * D;
    lse_g = a.lse2 + (int64_t)hq * a.t_q + it.q_base;
    drow_g = a.drow + (int64_t)hq * a.t_q + it.q_base;
  };
  const int kb0 = it.block * BN;          // first key of the block (sequence-local)
  const int kw = kb0 + 32 * w + c;        // this lane's key
  const int lo = it.tiles[0] & 0xffff, hi = (it.tiles[0] >> 16) & 0xffff;
  const int flo = it.full[0] & 0xffff, fhi = (it.full[0] >> 16) & 0xffff;
  const float c2 = a.scale_log2;
  const int wd = w % NDB;                 // head-dim block of this wave's dQ
  const int ld4 = (int)(ld * 4);          // dq_acc row stride in bytes
  const int dq_lane_off = (4 * h * (int)ld + 32 * wd + c) * 4;

  // fp32: K, V fragments in registers, lane (column kw) holds K[kw][KSTEP*t + h].
  op_t kf[kKVlds ? 1 : DSTEPS], vf[kKVlds ? 1 : DSTEPS];
  if constexpr (!kKVlds) {
    const bool ok = kw < it.skv;
    const int64_t off = (int64_t)(ok ? kw : 0) * ldkv;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
      kf[t] = ok ? M::load(kg + off + KSTEP * t + KPL * h) : op_t{};
      vf[t] = ok ? M::load(vg + off + KSTEP * t + KPL * h) : op_t{};
    }
  }

  floatx16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = floatx16{};
    dv[db] = floatx16{};
  }

  // Q / dY tiles straight to LDS; lse2 / D rows (and, with dropout, the keep
  // bits: thread (row = tid % BM, word = tid / BM) takes keys 32 word ..
  // 32 word + 31 of the block) through registers.
  float sreg = 0.f;
  uint32_t mreg[2] = {0u, 0u}, msh = 0;
  auto load_qtile = [&](int tile, int b) {
    const int nvalid = it.sq - tile * BM;
    tile_load_lds<T, D, BM>(qg + (int64_t)tile * BM * ld, ld, nvalid, qbuf + b * QTB, tid);
    tile_load_lds<T, D, BM>(dyg + (int64_t)tile * BM * ld, ld, nvalid, ybuf + b * QTB, tid);
    if (tid < 2 * BM) {
      const int row = tid & (BM - 1), i = tile * BM + row;
      if (tid < BM)
        sreg = i < it.sq ? lse_g[i] : INFINITY;
      else
        sreg = i < it.sq ? drow_g[i] : 0.f;
    }
    if constexpr (kDrop) {
      if (tid < 4 * BM) {
        const int row = tid & (BM - 1), i = tile * BM + row;
        const int64_t bit = drop_head + (int64_t)i * it.skv + kb0 + 32 * (tid / BM);
        const int64_t wd = bit >> 5;
        msh = (uint32_t)(bit & 31);
        mreg[0] = (i < it.sq && wd < a.drop.n_words) ? a.drop.words[wd] : 0u;
        mreg[1] = (i < it.sq && wd + 1 < a.drop.n_words) ? a.drop.words[wd + 1] : 0u;
      }
    }
  };
  auto store_rows = [&](int b) {
    if (tid < BM)
      lse_s[b][tid] = sreg;
    else if (tid < 2 * BM)
      drow_s[b][tid - BM] = sreg;
    if constexpr (kDrop) {
      if (tid < 4 * BM)
        mask_s[b * 4 * BM + (tid / BM) * BM + (tid & (BM - 1))] =
            __builtin_amdgcn_alignbit(mreg[1], mreg[0], msh);
    }
  };

  // Phase A for one query tile: P, dS, dV^T += dY^T P, dK^T += Q^T dS, dS -> LDS.
  auto phase_a = [&](auto mask_tag, int tile, int b) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const char* qt = qbuf + b * QTB;
    const char* yt = ybuf + b * QTB;
#pragma unroll 1
    for (int qb = 0; qb < QB; ++qb) {
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        // A: query rows of Q / dY; B: this lane's key row of K / V (all in LDS)
        const int off = tile_off<RB>(32 * qb + c, (KSTEP * t + KPL * h) * ES);
        op_t kb, vb;
        if constexpr (kKVlds) {
          const int koff = tile_off<RB>(32 * w + c, (KSTEP * t + KPL * h) * ES);
          kb = M::load(reinterpret_cast<const T*>(kblk + koff));
          vb = M::load(reinterpret_cast<const T*>(vblk + koff));
        } else {
          kb = kf[t];
          vb = vf[t];
        }
        s = M::mma(M::load(reinterpret_cast<const T*>(qt + off)), kb, s);
        dp = M::mma(M::load(reinterpret_cast<const T*>(yt + off)), vb, dp);
      }
      if constexpr (kKVlds) interleave_lds_mfma<2 * DSTEPS, 2, 2>();
      // rows of this lane: 32*qb + c_row(r, h); P = exp2(s*c - lse2), dS = P (dP - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb = 32 * qb + 8 * g + 4 * h;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[b][rb]);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&drow_s[b][rb]);
        uint32_t m4[4] = {0u, 0u, 0u, 0u};  // keep words of rows rb .. rb + 3, this wave's keys
        if constexpr (kDrop) {
#pragma unroll
          for (int e = 0; e < 4; ++e) m4[e] = mask_s[b * 4 * BM + w * BM + rb + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l4[e]));
          if constexpr (kMask)
            p = allowed(tile * BM + rb + e, kw, it.sq, it.skv, a.mode, it.band[0], it.band[1]) ? p : 0.f;
          if constexpr (kDrop) {
            // dV takes P Z / kp, dS = P (Z dP / kp - D)
            const bool kept = (m4[e] >> c) & 1u;
            dp[r] = p * ((kept ? dp[r] * a.drop.rkp : 0.f) - d4[e]);
            s[r] = kept ? p * a.drop.rkp : 0.f;
          } else {
            s[r] = p;
            dp[r] = p * (dp[r] - d4[e]);
          }
        }
      }
      // dV^T += dY^T P ;  dK^T += Q^T dS   (contraction over the 32 query rows)
#pragma unroll
      for (int t2 = 0; t2 < QSTEPS; ++t2) {
        const op_t pb = M::pack(s, t2);
        const op_t sb = M::pack(dp, t2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          op_t ya, qa;
          if constexpr (sizeof(T) == 2) {
            ya = tr_operand<RB, true>(yt, 32 * qb + KSTEP * t2, db, lane);
            qa = tr_operand<RB, true>(qt, 32 * qb + KSTEP * t2, db, lane);
          } else {
            const int row = 32 * qb + row_of_slot<T>(KSTEP * t2 + KPL * h);
            const int off = tile_off<RB>(row, (32 * db + c) * ES);
            ya = *reinterpret_cast<const T*>(yt + off);
            qa = *reinterpret_cast<const T*>(qt + off);
          }
          dv[db] = M::mma(ya, pb, dv[db]);
          dk[db] = M::mma(qa, sb, dk[db]);
        }
      }
      // dS (rounded to the input type) for the dQ product
      if constexpr (sizeof(T) == 2) {
        // Adjacent lanes hold adjacent keys of the same rows: swap one value
        // with the neighbour lane so that each lane stores a pair of keys of
        // one row as a single 32-bit word (even lanes rows r, odd lanes r+1).
        const bool odd = c & 1;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint32_t mine_r = __builtin_bit_cast(uint16_t, static_cast<T>(dp[r]));
          const uint32_t mine_r1 = __builtin_bit_cast(uint16_t, static_cast<T>(dp[r + 1]));
          const uint32_t give = odd ? mine_r : mine_r1;
          const uint32_t got = __builtin_amdgcn_mov_dpp((int)give, 0xB1, 0xF, 0xF, false);
          const uint32_t word = odd ? (got | (mine_r1 << 16)) : (mine_r | (got << 16));
          const int row = 32 * qb + c_row(odd ? r + 1 : r, h);
          *reinterpret_cast<uint32_t*>(sbuf + tile_off<SRB>(row, (32 * w + (c & ~1)) * ES)) = word;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          *reinterpret_cast<T*>(sbuf + tile_off<SRB>(32 * qb + c_row(r, h), (32 * w + c) * ES)) =
              static_cast<T>(dp[r]);
      }
    }
  };

  for (int gi = 0; gi < G; ++gi) {
    set_head(kvh * G + gi);
    if (lo <= hi) {
      if (gi == 0) {
        tile_load_lds<T, D, BN>(kg + (int64_t)kb0 * ldkv, ldkv, it.skv - kb0, kblk, tid);
        if constexpr (kKVlds)
          tile_load_lds<T, D, BN>(vg + (int64_t)kb0 * ldkv, ldkv, it.skv - kb0, vblk, tid);
      }
      load_qtile(lo, 0);
      store_rows(0);
      wait_vmem();
      __syncthreads();
    }
    for (int tile = lo; tile <= hi; ++tile) {
      const int b = (tile - lo) & 1;
      if (tile < hi) load_qtile(tile + 1, b ^ 1);
      if (tile < flo || tile > fhi)
        phase_a(std::true_type{}, tile, b);
      else
        phase_a(std::false_type{}, tile, b);
      __syncthreads();

      // dQ[32 rows x 32 d] = dS[rows, 128 keys] K[128 keys, d-block wd]
      const int nrows = it.sq - tile * BM < BM ? it.sq - tile * BM : BM;
      const bool full_rows = nrows == BM;
      const __amdgpu_buffer_rsrc_t dq_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          a.dq_acc + ((int64_t)it.q_base + tile * BM) * ld + head * D, (short)0,
          (int)(((int64_t)(nrows - 1) * ld + D) * 4), 0x00020000);
  #pragma unroll
      for (int k = 0; k < TASKS; ++k) {
        const int qb = w / NDB + k * WPD;
        floatx16 acc = floatx16{};
  #pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
          const op_t sa = M::load(reinterpret_cast<const T*>(
              sbuf + tile_off<SRB>(32 * qb + c, (KSTEP * t + KPL * h) * ES)));
          op_t kb;
          if constexpr (sizeof(T) == 2)
            kb = tr_operand<RB, false>(kblk, KSTEP * t, wd, lane);
          else
            kb = *reinterpret_cast<const T*>(kblk + tile_off<RB>(KSTEP * t + h, (32 * wd + c) * ES));
          acc = M::mma(sa, kb, acc);
        }
        // buffer atomics: wave-uniform row offset in an SGPR, one lane offset
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = tile * BM + 32 * qb + c_row(r, h);
          const int soff = (32 * qb + 8 * (r >> 2) + (r & 3)) * ld4;
          if (full_rows || i < it.sq)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], dq_rsrc, dq_lane_off, soff, 0);
        }
      }
      if (tile < hi) store_rows(b ^ 1);
      wait_vmem();
      __syncthreads();
    }

  }  // query heads of the group

  // epilogue: this lane's key column of dK^T / dV^T
  if (kw < it.skv) {
    const int64_t tok = (int64_t)it.kv_base + kw;
    T* dkp = static_cast<T*>(a.dk) + tok * ldkv + kvh * D;
    T* dvp = static_cast<T*>(a.dv) + tok * ldkv + kvh * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        if constexpr (sizeof(T) == 2) {
          bf16x4 k4, v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            k4[e] = static_cast<bf16>(dk[db][4 * g + e] * a.scale);
            v4[e] = static_cast<bf16>(dv[db][4 * g + e]);
          }
          *reinterpret_cast<bf16x4*>(dkp + d0) = k4;
          *reinterpret_cast<bf16x4*>(dvp + d0) = v4;
        } else {
          floatx4 k4, v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            k4[e] = dk[db][4 * g + e] * a.scale;
            v4[e] = dv[db][4 * g + e];
          }
          *reinterpret_cast<floatx4*>(dkp + d0) = k4;
          *reinterpret_cast<floatx4*>(dvp + d0) = v4;
        }
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void swa_dq_finalize_kernel(FinalizeArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= a.n) return;
  const floatx4 x0 = *reinterpret_cast<const floatx4*>(a.dq_acc + i);
  const floatx4 x1 = *reinterpret_cast<const floatx4*>(a.dq_acc + i + 4);
  T* out = static_cast<T*>(a.dq) + i;
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = static_cast<bf16>(x0[e] * a.scale);
      v[4 + e] = static_cast<bf16>(x1[e] * a.scale);
    }
    *reinterpret_cast<bf16x8*>(out) = v;
  } else {
    *reinterpret_cast<floatx4*>(out) = x0 * a.scale;
    *reinterpret_cast<floatx4*>(out + 4) = x1 * a.scale;
  }
}

__global__ __launch_bounds__(256) void swa_fill_kernel(FillArgs a) {
  const int64_t row_vecs = a.row_elems * a.elem_bytes / 16;
  const int64_t total = (a.row1 - a.row0) * row_vecs;
  uint8_t* base = static_cast<uint8_t*>(a.x) + a.row0 * a.row_elems * a.elem_bytes;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256)
    reinterpret_cast<Vec16*>(base)[i] = zero16();
  if (a.smax) {
    const int64_t stats = (a.row1 - a.row0) * a.stat_row;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < stats;
         i += (int64_t)gridDim.x * 256) {
      a.smax[a.row0 * a.stat_row + i] = -INFINITY;
      a.ssum[a.row0 * a.stat_row + i] = 0.f;
    }
  }
}

template <typename T, int D>
static int launch_pre_t(const BwdPreArgs& a, void* stream) {
  constexpr int RPB = 256 / (D / (16 / sizeof(T)));
  const int64_t nwg = (a.rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((swa_bwd_pre_kernel<T, D>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_pre(const BwdPreArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return head_dim == 128 ? launch_pre_t<bf16, 128>(a, stream)
                                         : launch_pre_t<bf16, 64>(a, stream);
  return head_dim == 128 ? launch_pre_t<float, 128>(a, stream)
                         : launch_pre_t<float, 64>(a, stream);
}

template <typename T, int D, bool kDrop>
static int launch_bwd_t(const BwdArgs& a, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_kv_heads;  // one workgroup per key block and K/V head
  constexpr int BM = bwd_block_q(sizeof(T) == 2 ? 1 : 0, D);
  hipLaunchKernelGGL((swa_bwd_kernel<T, D, BM, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_backward(const BwdArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return launch_bwd_kv(a, head_dim, stream);  // swa_bwd_kv.hip
  if (a.drop.words)
    return head_dim == 128 ? launch_bwd_t<float, 128, true>(a, stream)
                           : launch_bwd_t<float, 64, true>(a, stream);
  return head_dim == 128 ? launch_bwd_t<float, 128, false>(a, stream)
                         : launch_bwd_t<float, 64, false>(a, stream);
}

int launch_dq_finalize(const FinalizeArgs& a, int dtype, void* stream) {
  const int64_t nwg = (a.n / 8 + 255) / 256;
  if (nwg == 0) return 0;
  if (dtype == 1)
    hipLaunchKernelGGL((swa_dq_finalize_kernel<bf16>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_dq_finalize_kernel<float>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_fill(const FillArgs& a, void* stream) {
  const int64_t total = (a.row1 - a.row0) * a.row_elems * a.elem_bytes / 16;
  int64_t nwg = (total + 255) / 256;
  if (nwg < 1) nwg = 1;
  if (nwg > 4096) nwg = 4096;
  hipLaunchKernelGGL(swa_fill_kernel, dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

const char* hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

int hip_memcpy_h2d_async(void* dst, const void* src, size_t bytes, void* stream) {
  return (int)hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice,
                             static_cast<hipStream_t>(stream));
}
int hip_pinned_alloc(void** p, size_t bytes) { return (int)hipHostMalloc(p, bytes, hipHostMallocDefault); }
int hip_pinned_free(void* p) { return (int)hipHostFree(p); }
int hip_event_create(void** ev) {
  return (int)hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(ev), hipEventDisableTiming);
}
int hip_event_record(void* ev, void* stream) {
  return (int)hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream));
}
int hip_event_sync(void* ev) { return (int)hipEventSynchronize(static_cast<hipEvent_t>(ev)); }
int hip_event_create_timed(void** ev) {
  return (int)hipEventCreate(reinterpret_cast<hipEvent_t*>(ev));
}
int hip_event_elapsed_ms(float* ms, void* start, void* stop) {
  return (int)hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
}
int hip_event_destroy(void* ev) { return (int)hipEventDestroy(static_cast<hipEvent_t>(ev)); }

int hip_stream_device(void* stream, int* dev) {
  const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), dev)
                              : hipGetDevice(dev);
  return (int)e;
}

namespace {
// Run f with `device` current, restoring the caller's device afterwards.
template <typename F>
int on_device(int device, F&& f) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return (int)e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return (int)e;
  e = f();
  if (cur != device) {
    const hipError_t r = hipSetDevice(cur);
    if (e == hipSuccess) e = r;
  }
  return (int)e;
}
}  // namespace

int hip_device_alloc(int device, void** p, size_t bytes) {
  return on_device(device, [&] { return hipMalloc(p, bytes); });
}
int hip_device_free(int device, void* p) {
  return on_device(device, [&] {
    const hipError_t e = hipDeviceSynchronize();
    return e != hipSuccess ? e : hipFree(p);
  });
}
int hip_memcpy_h2d_sync(int device, void* dst, const void* src, size_t bytes) {
  return on_device(device, [&] { return hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice); });
}

int hip_cu_count(void* stream, int* n) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                        : hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return (int)e;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  *n = v;
  return 0;
}

}  // namespace swa
