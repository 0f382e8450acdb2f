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
// Both input types run the two-pass structure of the PyPTO-Gym article
// (两趟循环结构): a KV-outer pass for dK, dV and a Q-outer pass for dQ, P and
// dS recomputed in both, with no atomics, so every output is bitwise
// reproducible (the deterministic mode of the explainer, section 6.1).
// bf16: swa_bwd_dq_kernel (dQ; it also forms D and lse2, in swa_bwd_dq.hip),
//   then swa_bwd_kv_kernel (dK, dV, in swa_bwd_kv.hip).
// fp32 (this file):
//   swa_bwd_pre_kernel: D and the per-row log2-domain normaliser
//     lse2 = softmax_max * log2(e) + log2(softmax_sum), so that
//     P = exp2(s*c - lse2) with c = scale * log2(e);
//   swa_bwd_kv_f32_kernel: one workgroup per (block of 128 keys, head); each
//     of its 4 waves owns 32 keys, keeps their K and V rows and its dK, dV
//     accumulators in registers and walks the query tiles of the band.
//     Scores are formed as S = Q K^T (queries as rows, the wave's keys as
//     columns), so P and dS come out of the accumulators in the operand
//     layout of dV^T += dY^T P and dK^T += Q^T dS.  Q and dY tiles go from
//     HBM straight into swizzled row-major LDS tiles (double-buffered, rows
//     past the sequence read as zero).  With grouped heads the workgroup of a
//     key/value head walks the query heads of its group in turn; with
//     dropout the keep bits of each query tile are staged in LDS next to
//     lse2 and D;
//   swa_bwd_dq_f32_kernel: one workgroup per (block of 128 query rows,
//     head); a lane owns one query row (its Q and dY rows in registers as B
//     operands of S^T = K Q^T and dP^T = V dY^T, its lse2 and D as scalars)
//     and its column of dQ^T += K^T dS^T, over the key tiles of the band.

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "swa_common.hpp"

namespace swa {

template <typename T, int D>
__global__ __launch_bounds__(256) void swa_bwd_pre_kernel(BwdPreArgs a) {
  static_assert(sizeof(T) == 4, "fp32 inputs (bf16 forms D in its dQ kernel)");
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
  if (ch == 0) {
    const int64_t tok = row / a.num_heads, head = row - tok * a.num_heads;
    const int64_t at = head * a.t_q + tok;  // head-major so that a tile's rows are contiguous
    a.drow[at] = acc;
    const float mx = a.smax[row * 8], sm = a.ssum[row * 8];
    a.lse2[at] = (sm > 0.f && mx > -INFINITY) ? mx * 1.4426950408889634f + log2f(sm) : INFINITY;
  }
}

template <int D, int BM, bool kDrop>
__global__ __launch_bounds__(256, 1) void swa_bwd_kv_f32_kernel(BwdArgs a) {
  using T = float;
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int BN = BWD_BN;
  constexpr int ES = (int)sizeof(T);
  constexpr int RB = D * ES;              // Q / dY tile row bytes
  constexpr int QTB = BM * RB;            // Q or dY tile bytes
  constexpr int NDB = D / 32;             // head-dim blocks
  constexpr int QB = BM / 32;             // 32-row query blocks per tile
  constexpr int DSTEPS = D / KSTEP;       // contraction steps over d
  constexpr int QSTEPS = 32 / KSTEP;      // contraction steps per 32 query rows
  static_assert(BN == 128 && (BM == 64 || BM == 32), "4 waves x 32 keys; 32/64-row tiles");

  __shared__ __attribute__((aligned(1024))) char lds[4 * QTB];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BM];
  __shared__ __attribute__((aligned(16))) float drow_s[2][BM];
  // dropout keep bits of the tile: [slot][key word kw / 32 of the block][row]
  __shared__ __attribute__((aligned(16))) uint32_t mask_s[kDrop ? 2 * 4 * BM : 1];
  // slot b: the Q tile at lds + 2 QTB b, its dY tile right after it
  char* const qbuf = lds;
  char* const ybuf = lds + QTB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kvh = L / a.n_items;  // the grid runs over key/value heads
  const Item it = a.items[L - kvh * a.n_items];
  const int N = a.num_heads;
  const int G = N / a.num_kv_heads;                  // query heads sharing this K / V
  const int64_t ld = (int64_t)N * D;                 // q / dy row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v / dk / dv row stride
  const T* kg = static_cast<const T*>(a.k) + (int64_t)it.kv_base * ldkv + kvh * D;
  const T* vg = static_cast<const T*>(a.v) + (int64_t)it.kv_base * ldkv + kvh * D;
  // the query head being processed (the group's heads run one after another,
  // accumulating into the same dK / dV) and its tensors
  const T* qg = nullptr;
  const T* dyg = nullptr;
  const float* lse_g = nullptr;
  const float* drow_g = nullptr;
  int64_t drop_head = 0;  // first dropout-mask bit of (sequence, query head)
  auto set_head = [&](int hq) {
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

  // K, V fragments in registers, lane (column kw) holds K[kw][KSTEP*t + h].
  op_t kf[DSTEPS], vf[DSTEPS];
  {
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
    tile_load_lds<T, D, BM>(qg + (int64_t)tile * BM * ld, ld, nvalid, qbuf + 2 * b * QTB, tid);
    tile_load_lds<T, D, BM>(dyg + (int64_t)tile * BM * ld, ld, nvalid, ybuf + 2 * b * QTB, tid);
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

  // One query tile: P, dS, dV^T += dY^T P, dK^T += Q^T dS.
  auto tile_step = [&](auto mask_tag, int tile, int b) {
    constexpr bool kMask = decltype(mask_tag)::value;
    const char* qt = qbuf + 2 * b * QTB;
    const char* yt = ybuf + 2 * b * QTB;
#pragma unroll 1
    for (int qb = 0; qb < QB; ++qb) {
      // lane indices formed here, per block (an empty asm keeps the compiler
      // from hoisting the many LDS offsets below out of the loops, which
      // would keep them all live in registers)
      int ln = tid;
      asm volatile("" : "+v"(ln));
      const int h = (ln >> 5) & 1, c = ln & 31;
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        // A: query rows of Q / dY (LDS); B: this lane's key row of K / V (registers)
        const int off = tile_off<RB>(32 * qb + c, (KSTEP * t + KPL * h) * ES);
        s = M::mma(M::load(reinterpret_cast<const T*>(qt + off)), kf[t], s);
        dp = M::mma(M::load(reinterpret_cast<const T*>(yt + off)), vf[t], dp);
      }
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
          const int row = 32 * qb + row_of_slot<T>(KSTEP * t2 + KPL * h);
          const int off = tile_off<RB>(row, (32 * db + c) * ES);
          dv[db] = M::mma(*reinterpret_cast<const T*>(yt + off), pb, dv[db]);
          dk[db] = M::mma(*reinterpret_cast<const T*>(qt + off), sb, dk[db]);
        }
      }
    }
  };

  for (int gi = 0; gi < G; ++gi) {
    set_head(kvh * G + gi);
    if (lo <= hi) {
      load_qtile(lo, 0);
      store_rows(0);
      wait_vmem();
      __syncthreads();
    }
    for (int tile = lo; tile <= hi; ++tile) {
      const int b = (tile - lo) & 1;
      if (tile < hi) load_qtile(tile + 1, b ^ 1);
      if (tile < flo || tile > fhi)
        tile_step(std::true_type{}, tile, b);
      else
        tile_step(std::false_type{}, tile, b);
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

template <int D, bool kDrop>
__global__ __launch_bounds__(256, 1) void swa_bwd_dq_f32_kernel(BwdArgs a) {
  using M = Mfma<float>;
  constexpr int BQ = 128;          // query rows per workgroup
  constexpr int BN = FWD_BN;       // keys per tile
  constexpr int RB = D * 4;        // row bytes
  constexpr int KTB = BN * RB;     // K or V tile bytes
  constexpr int NDB = D / 32;      // head-dim blocks
  constexpr int DSTEPS = D / 2;    // contraction steps over d (2 per step)
  static_assert(BN == 64, "two 32-key blocks per tile");
  __shared__ __attribute__((aligned(1024))) char lds[4 * KTB];  // K[2] | V[2]
  char* const kbuf = lds;
  char* const vbuf = lds + 2 * KTB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.n_items;
  const Item it = a.items[L - head * a.n_items];
  const int64_t ld = (int64_t)a.num_heads * D;       // q / dy / dq row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v row stride
  const int kvh = head / (a.num_heads / a.num_kv_heads);  // grouped heads share K / V
  const float* kg = static_cast<const float*>(a.k) + (int64_t)it.kv_base * ldkv + kvh * D;
  const float* vg = static_cast<const float*>(a.v) + (int64_t)it.kv_base * ldkv + kvh * D;
  const int qrow = it.block * BQ + 32 * w + c;  // this lane's query row (sequence-local)
  const bool row_ok = qrow < it.sq;
  const int lo = it.tiles[0] & 0xffff, hi = (it.tiles[0] >> 16) & 0xffff;
  const float c2 = a.scale_log2;

  // B operands of S^T = K Q^T and dP^T = V dY^T: lane (column qrow) holds
  // Q[qrow][2t + h], dY likewise; the row's lse2 and D
  float qf[DSTEPS], yf[DSTEPS];
  {
    const int64_t off = ((int64_t)it.q_base + (row_ok ? qrow : 0)) * ld + head * D;
    const float* qp = static_cast<const float*>(a.q) + off;
    const float* yp = static_cast<const float*>(a.dy) + off;
#pragma unroll
    for (int t4 = 0; t4 < D / 4; ++t4) {
      const floatx4 q4 = *reinterpret_cast<const floatx4*>(qp + 4 * t4);
      const floatx4 y4 = *reinterpret_cast<const floatx4*>(yp + 4 * t4);
      qf[2 * t4] = row_ok ? q4[h] : 0.f;
      qf[2 * t4 + 1] = row_ok ? q4[2 + h] : 0.f;
      yf[2 * t4] = row_ok ? y4[h] : 0.f;
      yf[2 * t4 + 1] = row_ok ? y4[2 + h] : 0.f;
    }
  }
  const int64_t at = (int64_t)head * a.t_q + it.q_base + (row_ok ? qrow : 0);
  const float lse = row_ok ? a.lse2[at] : INFINITY;  // rows past the end: P = 0
  const float drow = row_ok ? a.drow[at] : 0.f;
  // keys allowed for this lane's row: j in [j_min, j_max]
  int j_min = 0, j_max = it.skv - 1;
  if (a.mode != 0) {  // (the item's band is clamped to +-2^30 and qrow < 2^20: no overflow)
    const int lo32 = qrow - it.band[0], hi32 = qrow + it.band[1];
    j_min = lo32 < 0 ? 0 : (lo32 > it.skv ? it.skv : lo32);
    j_max = hi32 < j_max ? (hi32 < -1 ? -1 : hi32) : j_max;
  }
  if (!row_ok) j_max = -1;
  const int64_t drop_row = kDrop ? it.drop_base + (int64_t)head * it.sq * it.skv +
                                       (int64_t)(row_ok ? qrow : 0) * it.skv
                                 : 0;

  auto load_tile = [&](int tile, int b) {
    tile_load_lds<float, D, BN>(kg + (int64_t)tile * BN * ldkv, ldkv, it.skv - tile * BN,
                                kbuf + b * KTB, tid);
    tile_load_lds<float, D, BN>(vg + (int64_t)tile * BN * ldkv, ldkv, it.skv - tile * BN,
                                vbuf + b * KTB, tid);
  };

  floatx16 acc[NDB];  // dQ^T: rows = head dim 32 db + c_row(r, h), column = this lane's row
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
  if (lo <= hi) {
    load_tile(lo, 0);
    wait_vmem();
    __syncthreads();
  }
  for (int tile = lo; tile <= hi; ++tile) {
    const int b = (tile - lo) & 1;
    if (tile < hi) load_tile(tile + 1, b ^ 1);
    const char* kt = kbuf + b * KTB;
    const char* vt = vbuf + b * KTB;
    // keep bits of this lane's row for the tile's 64 keys (bit k = key 64 tile + k)
    uint32_t keep[2] = {0u, 0u};
    if constexpr (kDrop) {
      const int64_t bit = drop_row + (int64_t)tile * BN, wd = bit >> 5;
      uint32_t mw[3];
#pragma unroll
      for (int e = 0; e < 3; ++e) mw[e] = (row_ok && wd + e < a.drop.n_words) ? a.drop.words[wd + e] : 0u;
      const uint32_t sh = (uint32_t)(bit & 31);
      keep[0] = __builtin_amdgcn_alignbit(mw[1], mw[0], sh);
      keep[1] = __builtin_amdgcn_alignbit(mw[2], mw[1], sh);
    }
#pragma unroll 1
    for (int jb = 0; jb < 2; ++jb) {
      // S^T, dP^T of keys 32 jb + c_row(r, h) (rows) and this lane's query (column)
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        const int off = tile_off<RB>(32 * jb + c, (2 * t + h) * 4);
        s = M::mma(*reinterpret_cast<const float*>(kt + off), qf[t], s);
        dp = M::mma(*reinterpret_cast<const float*>(vt + off), yf[t], dp);
      }
      // P = exp2(s c - lse2), masked; dS = P (dP - D) (with dropout, P (Z dP / kp - D))
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jt = 32 * jb + c_row(r, h);  // key within the tile
        const int j = tile * BN + jt;
        float p = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lse));
        p = (j >= j_min && j <= j_max) ? p : 0.f;
        if constexpr (kDrop) {
          const bool kept = (keep[jb] >> c_row(r, h)) & 1u;
          dp[r] = p * ((kept ? dp[r] * a.drop.rkp : 0.f) - drow);
        } else {
          dp[r] = p * (dp[r] - drow);
        }
      }
      // dQ^T += K^T dS^T: step t2 takes dS^T register t2, the key c_row(t2, h)
      // of the block, so the K^T operand of lane l is K[that key][32 db + l % 32]
#pragma unroll
      for (int t2 = 0; t2 < 16; ++t2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float ka = *reinterpret_cast<const float*>(
              kt + tile_off<RB>(32 * jb + c_row(t2, h), (32 * db + c) * 4));
          acc[db] = M::mma(ka, dp[t2], acc[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
  // dq = scale dQ (zero for a row that attends no key)
  if (row_ok) {
    float* op = static_cast<float*>(a.dq) + ((int64_t)it.q_base + qrow) * ld + head * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[db][4 * g + e] * a.scale;
        *reinterpret_cast<floatx4*>(op + 32 * db + 8 * g + 4 * h) = v4;
      }
    }
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

template <int D>
static int launch_pre_t(const BwdPreArgs& a, void* stream) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t nwg = (a.rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((swa_bwd_pre_kernel<float, D>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_pre(const BwdPreArgs& a, int head_dim, void* stream) {
  return head_dim == 128 ? launch_pre_t<128>(a, stream) : launch_pre_t<64>(a, stream);
}

template <int D, bool kDrop>
static int launch_kv_f32_t(const BwdArgs& a, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_kv_heads;  // one workgroup per key block and K/V head
  hipLaunchKernelGGL((swa_bwd_kv_f32_kernel<D, BWD_BM, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_backward(const BwdArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return launch_bwd_kv(a, head_dim, stream);  // swa_bwd_kv.hip
  if (a.drop.words)
    return head_dim == 128 ? launch_kv_f32_t<128, true>(a, stream)
                           : launch_kv_f32_t<64, true>(a, stream);
  return head_dim == 128 ? launch_kv_f32_t<128, false>(a, stream)
                         : launch_kv_f32_t<64, false>(a, stream);
}

template <int D, bool kDrop>
static int launch_dq_f32_t(const BwdArgs& a, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_heads;  // one workgroup per query block and head
  hipLaunchKernelGGL((swa_bwd_dq_f32_kernel<D, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_dq_f32(const BwdArgs& a, int head_dim, void* stream) {
  if (a.drop.words)
    return head_dim == 128 ? launch_dq_f32_t<128, true>(a, stream)
                           : launch_dq_f32_t<64, true>(a, stream);
  return head_dim == 128 ? launch_dq_f32_t<128, false>(a, stream)
                         : launch_dq_f32_t<64, false>(a, stream);
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
