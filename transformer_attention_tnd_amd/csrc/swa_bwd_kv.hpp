// The bf16 dK/dV kernel template (the KV-outer pass of the two-pass
// backward).  Instantiated in swa_bwd_kv.hip (one query head per key/value
// head, compiled with the matrix-core results in ordinary vector registers,
// so the softmax reads the S and dP accumulators without copies) and in
// swa_bwd_kv_gqa.hip (grouped heads).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "swa_common.hpp"
#include "swa_pipe.hpp"

namespace swa {

// bf16 backward in two kernels, no atomics (deterministic): the two-pass
// structure of the PyPTO-Gym FlashAttentionScoreGrad article (两趟循环结构),
// which recomputes P and dS in both passes.
//   swa_bwd_kv_kernel: one workgroup per (block of 128 keys, head); each of
//     its 4 waves owns 32 keys, keeps its K and V rows in registers (B
//     operands of S = Q K^T and dP = dY V^T) and its dK^T, dV^T accumulators,
//     and walks the query tiles (64 rows) of the band.
//   swa_bwd_dq_kernel: one workgroup per (block of 128 query rows, head);
//     each wave owns 32 rows, keeps its Q and dY rows in registers (B operands
//     of S^T = K Q^T and dP^T = V dY^T) and its dQ^T accumulator, and walks the
//     key tiles (64 keys) of the band; dQ^T += K^T dS^T takes K^T from the
//     key tile through transposing LDS reads.  dq is written once, in the
//     input type.  It runs first and also forms D = rowsum(dY o O) and lse2
//     of its rows, which this kernel reads (D stored negated: without dropout
//     the dP chains here start from -D).
// Both are persistent: one workgroup per compute unit runs a list of
// (item, head) units from the host (see swa_host.cpp, build_worklist).
// Both are organised for one wave per SIMD.  The products of a tile form one
// software pipeline in a fixed order; each LDS operand is read a fixed number
// of products ahead into a small register ring, and the vector work (the
// softmax elements) is spread over the slots between products, with
// scheduling fences keeping that order.  LDS holds two slabs (the tiles of
// query/key tile t and t+1, copied straight from HBM by instructions that the
// pipeline of tile t issues one every few slots, so that the copies do not
// stall the waves in a burst); the lane offsets into them sit in registers
// and move to the other slab once per tile.
template <int D, bool kGroups, bool kDrop>
__global__ __launch_bounds__(256, 1) void swa_bwd_kv_kernel(BwdArgs a) {
  using M = Mfma<bf16>;
  using op_t = M::op_t;
  constexpr int BN = BWD_BN;           // keys per workgroup
  constexpr int BM = 64;               // query rows per tile
  constexpr int RB = D * 2;            // row bytes
  constexpr int QTB = BM * RB;         // Q or dY tile bytes
  constexpr int SLAB = 2 * QTB;        // Q | dY
  constexpr int NDB = D / 32;          // head-dim blocks
  constexpr int DSTEPS = D / 16;       // contraction steps over d
  // products of one tile, in issue order: S/dP of rows 0-31, of rows 32-63,
  // dV/dK of rows 0-31, of rows 32-63
  constexpr int NS = 2 * DSTEPS, NV = 4 * NDB;
  constexpr int G_S1 = NS, G_V0 = 2 * NS, G_V1 = G_V0 + NV, NOPS = G_V1 + NV;
  constexpr int AHEAD = SWA_BWD_AHEAD, RING = AHEAD + 1;
  constexpr int COPY_EVERY = 4;        // pipeline slots between copy instructions
  static_assert(BN == 128 && (D == 64 || D == 128), "4 waves x 32 keys, 64-row tiles");
  // Slot of the first softmax stage of register r of block qb: the 16
  // registers are spread evenly from the end of the block's S / dP products
  // to two slots before the dV / dK products that use registers 8..15;
  // registers 0..7 then finish before the products that use them.
  constexpr auto kv_soft_slot = [](int qb, int r) {
    const int rel = qb == 0 ? G_S1 : G_V0, last = (qb == 0 ? G_V0 : G_V1) + NV / 2 - 2;
    return rel + (r * (last - rel)) / 15;
  };
  static_assert(kv_soft_slot(0, 7) + 1 < G_V0 && kv_soft_slot(1, 7) + 1 < G_V1 &&
                kv_soft_slot(0, 15) + 1 < G_V0 + NV / 2 && kv_soft_slot(1, 15) + 1 < G_V1 + NV / 2,
                "softmax stages finish before the products that use them");

  // two slabs (Q | dY of tiles t and t + 1), then the epilogue area (the dK
  // and dV rows of the 4 waves), so that the slabs can take the next unit's
  // first tile while a unit's results leave
  constexpr int EPI = 2 * 4 * 32 * RB;
  __shared__ __attribute__((aligned(1024))) char lds[2 * SLAB + EPI];
  char* const epi = lds + 2 * SLAB;
  __shared__ floatx4 lse_s[2][BM / 4];   // lse2 of the tile's rows
  __shared__ floatx4 drow_s[2][BM / 4];  // -D of the tile's rows
  // dropout keep bits of the tile: [slot][key word kw / 32 of the block][row],
  // bit c of a word = key 32 * word + c
  __shared__ uint32_t mask_s[kDrop ? 2 * 4 * BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int32_t* work = a.work + a.work_off[blockIdx.x];
  const int n_units = a.work_off[blockIdx.x + 1] - a.work_off[blockIdx.x];
  if (n_units <= 0) return;
  // query heads sharing this K / V (kGroups == false: exactly one)
  const int G = kGroups ? a.num_heads / a.num_kv_heads : 1;
  const int64_t ld = (int64_t)a.num_heads * D;       // q / dy row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v / dk / dv row stride
  const float c2 = a.scale_log2;

  // the current unit (a block of BN keys of one key/value head)
  UnitInfo it;
  int kvh = 0;
  int lo = 1, hi = 0, flo = 1, fhi = 0;
  // the query head being processed (the group's heads run one after another,
  // accumulating into the same dK / dV registers) and its tensors
  const bf16* qg = nullptr;
  const bf16* dyg = nullptr;
  const float* lse_g = nullptr;
  const float* drow_g = nullptr;
  int64_t drop_head = 0;  // first dropout-mask bit of (sequence, query head)
  auto set_head = [&](int hq) {
    drop_head = it.drop_base + (int64_t)hq * it.sq * it.skv;
    qg = static_cast<const bf16*>(a.q) + (int64_t)it.q_base * ld + hq * D;
    dyg = static_cast<const bf16*>(a.dy) + (int64_t)it.q_base * ld + hq * D;
    lse_g = a.lse2 + (int64_t)hq * a.t_q + it.q_base;
    drow_g = a.drow + (int64_t)hq * a.t_q + it.q_base;
  };
  auto set_unit = [&](const UnitInfo& u) {
    it = u;
    kvh = u.head;
    lo = u.tiles0 & 0xffff;
    hi = (u.tiles0 >> 16) & 0xffff;
    flo = u.full0 & 0xffff;
    fhi = (u.full0 >> 16) & 0xffff;
  };
  int kw = 0;  // this lane's key (sequence-local)

  floatx16 dk[NDB], dv[NDB];
  // B operands of S and dP: lane (column kw) holds K[kw][16t + 8h + e], V likewise
  op_t kr[DSTEPS], vr[DSTEPS];
  auto load_kv_rows = [&](const UnitInfo& u) {
    const int key = u.block * BN + 32 * w + c;
    const bool ok = key < u.skv;
    const int64_t off = ((int64_t)u.kv_base + (ok ? key : 0)) * ldkv + u.head * D + 8 * h;
    const bf16* kp = static_cast<const bf16*>(a.k) + off;
    const bf16* vp = static_cast<const bf16*>(a.v) + off;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
      kr[t] = ok ? M::load(kp + 16 * t) : op_t{};
      vr[t] = ok ? M::load(vp + 16 * t) : op_t{};
    }
  };
  // Rows allowed for this lane's key: i in [i_min, i_max] (empty if the key
  // is past the sequence), from the band rule -pre <= kw - i <= next.
  int i_min = 0, i_max = -1;
  auto key_range = [&]() {
    kw = it.block * BN + 32 * w + c;
    i_min = 0;
    i_max = it.sq - 1;
    if (a.mode != 0) {  // 64-bit: pre / next may be near the int range
      const int64_t lo64 = (int64_t)kw - it.next, hi64 = (int64_t)kw + it.pre;
      i_min = lo64 < 0 ? 0 : (lo64 > it.sq ? it.sq : (int)lo64);
      i_max = hi64 < i_max ? (hi64 < -1 ? -1 : (int)hi64) : i_max;
    }
    if (kw >= it.skv) i_max = -1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk[db] = floatx16{};
      dv[db] = floatx16{};
    }
  };

  // Lane offsets (slab of the current tile).  Rows 16 apart share a swizzle,
  // so the 32-row block, the 16-row step and Q vs dY are immediate offsets.
  int oq[DSTEPS];   // 128-bit read of row c, chunk 2t + h
  int otr[NDB][2];  // transposing reads, head-dim block db
  int olr = 16 * h; // lse2 / D of rows 4h .. 4h + 3 of each 8
  int omk = (w * BM + 4 * h) * 4;  // keep words of this wave's keys, rows 4h .. 4h + 3 of each 8
#pragma unroll
  for (int t = 0; t < DSTEPS; ++t) oq[t] = tile_off<RB>(c, (16 * t + 8 * h) * 2);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_offsets<RB>(lane, db, otr[db][0], otr[db][1]);

  // dropout: thread (row = tid % 64, word = tid / 64) fetches the 32 keep bits
  // of its row for keys 32 word .. 32 word + 31 of the block (two words and a
  // shift, joined when they are stored)
  uint32_t mreg[2] = {0u, 0u}, msh = 0;
  // copies of the next tile's Q and dY into its slab, issued part by part
  // from the pipeline of the current tile; a tile past the band copies zeros
  // (no memory read) into the free slab
  using Dma = TileDma<bf16, D, BM>;
  Dma cp_q, cp_dy;
  auto start_copy = [&](int tile, int b) {
    const int nvalid = tile <= hi ? it.sq - tile * BM : 0;
    char* slab = lds + b * SLAB;
    cp_q.init(qg + (int64_t)tile * BM * ld, ld, nvalid, slab, tid);
    cp_dy.init(dyg + (int64_t)tile * BM * ld, ld, nvalid, slab + QTB, tid);
  };
  // lse2 / -D of the tile's rows go straight into LDS slot b (wave 0: lse2,
  // wave 1: -D; one 64-lane dword copy each, rows past the sequence read as
  // zero: the tiles that hold such rows are masked tiles, where their P is
  // zero whatever lse2 holds), waited for with the tile copies; with dropout
  // the keep bits of the rows go through registers (store_rows)
  // (of a unit with query length sq, key length skv, key block kb, whose
  // head's lse2 / -D rows start at lse_b / drow_b and keep bits at dh)
  auto load_rows_of = [&](const float* lse_b, const float* drow_b, int sq, int skv, int kb,
                          int64_t dh, int tile, int b) {
    if (w < 2) {
      const int nv = sq - tile * BM;
      const uint32_t nrec = nv <= 0 ? 0u : (uint32_t)(nv < BM ? nv : BM) * 4u;
      const float* src = (w == 0 ? lse_b : drow_b) + (int64_t)tile * BM;
      const uint32_t dst = lds_addr(w == 0 ? (const void*)lse_s[b] : (const void*)drow_s[b]);
      dma4(buffer_rsrc(src, nrec), (uint32_t)lane * 4u, __builtin_amdgcn_readfirstlane(dst));
    }
    if constexpr (kDrop) {
      const int row = tid & (BM - 1), i = tile * BM + row;
      const int64_t bit = dh + (int64_t)i * skv + kb * BN + 32 * (tid / BM);
      const int64_t wd = bit >> 5;
      msh = (uint32_t)(bit & 31);
      mreg[0] = (i < sq && wd < a.drop.n_words) ? a.drop.words[wd] : 0u;
      mreg[1] = (i < sq && wd + 1 < a.drop.n_words) ? a.drop.words[wd + 1] : 0u;
    }
  };
  auto load_rows = [&](int tile, int b) {
    load_rows_of(lse_g, drow_g, it.sq, it.skv, it.block, drop_head, tile, b);
  };
  // The next unit, prefetched by the pipeline of this unit's last tile (when
  // that tile is masked): its first query tile and rows into the free slab,
  // and its K / V rows into the epilogue area (read into registers at the
  // switch, before this unit's dK / dV pass through that area).
  using KvDma = TileDma<bf16, D, BN>;
  KvDma kv_st;     // K rows of the next unit (lane offsets, destination)
  u32x4 kv_v_rsrc;  // its V rows (same offsets, 32 rows x RB further on)
  struct Next {
    const float* lse_b;
    const float* drow_b;
    int sq, skv, block, lo;
    int64_t dh;
  } nx;
  auto prefetch_select = [&](const UnitInfo& n, int b) {
    const int hq = n.head * G;
    const int nlo = n.tiles0 & 0xffff, nhi = (n.tiles0 >> 16) & 0xffff;
    const bf16* q0 = static_cast<const bf16*>(a.q) + (int64_t)n.q_base * ld + hq * D;
    const bf16* y0 = static_cast<const bf16*>(a.dy) + (int64_t)n.q_base * ld + hq * D;
    const int nvalid = nlo <= nhi ? n.sq - nlo * BM : 0;
    char* slab = lds + b * SLAB;
    cp_q.init(q0 + (int64_t)nlo * BM * ld, ld, nvalid, slab, tid);
    cp_dy.init(y0 + (int64_t)nlo * BM * ld, ld, nvalid, slab + QTB, tid);
    nx.lse_b = a.lse2 + (int64_t)hq * a.t_q + n.q_base;
    nx.drow_b = a.drow + (int64_t)hq * a.t_q + n.q_base;
    nx.sq = n.sq;
    nx.skv = n.skv;
    nx.block = n.block;
    nx.lo = nlo;
    nx.dh = n.drop_base + (int64_t)hq * n.sq * n.skv;
    const int64_t ko = ((int64_t)n.kv_base + n.block * BN) * ldkv + n.head * D;
    kv_st.init(static_cast<const bf16*>(a.k) + ko, ldkv, n.skv - n.block * BN, epi, tid);
    kv_v_rsrc = buffer_rsrc(static_cast<const bf16*>(a.v) + ko, kv_st.rsrc[2]);
  };
  auto kv_stage_issue = [&](auto pc) {
    constexpr int pt = decltype(pc)::value;  // K parts, then V parts
    if constexpr (pt < KvDma::PARTS)
      kv_st.template issue<pt>();
    else
      dma16(kv_v_rsrc, kv_st.voff + (pt - KvDma::PARTS) * kv_st.vstep,
            kv_st.dst + BN * RB + (pt - KvDma::PARTS) * 256 * 16);
  };
  auto copy_all = [&]() {
    static_for<Dma::PARTS>([&](auto pc) {
      cp_q.template issue<decltype(pc)::value>();
      cp_dy.template issue<decltype(pc)::value>();
    });
  };
  auto store_rows = [&](int b) {
    if constexpr (kDrop)
      mask_s[b * 4 * BM + (tid / BM) * BM + (tid & (BM - 1))] =
          __builtin_amdgcn_alignbit(mreg[1], mreg[0], msh);
  };
  auto rd128 = [&](int off) { return *reinterpret_cast<const op_t*>(lds + off); };

  // One query tile: S, dP, P, dS, dV^T += dY^T P, dK^T += Q^T dS.
  // One query tile (slab b): also issues the copies of tile + 1 into slab b ^ 1
  auto step = [&](auto mask_tag, int tile, int b, auto next_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    // kNext: the last tile of the unit, which prefetches the next one
    constexpr bool kNext = decltype(next_tag)::value;
    // row 32 qb + 8 g + 4 h + e is allowed iff 32 qb + 8 g + e lies in the lane's range rg
    LaneRange rg{0, 0u};
    if constexpr (kMask) rg = lane_range(i_min - tile * BM - 4 * h, i_max - tile * BM - 4 * h, BM);
    op_t ring[RING];
    floatx16 s[2], dp[2];
    // lse2 and the stored row term -D of 4 rows (with dropout lse2 + log2(kp)
    // and -D kp, so that exp2(s c - lse2) = P / kp); dv4 is loaded when the
    // softmax needs it (grouped heads, dropout)
    floatx4 lv[2][4], dv4[2][4];
    floatx16 nd[2];  // the row term of the rows of accumulator registers 0..15 of block qb
    // The dP chain starts from the row term, so that the accumulator ends as
    // dP - D (dropout: dP - D kp) and dS = P (dP - D) is one multiply; with
    // dropout dS = P (Z dP / kp - D) = (P / kp) (Z ? dP - D kp : -D kp), a
    // select and one multiply, and dV takes P Z / kp.  Not in the grouped
    // build with dropout, compiled with the default register assignment,
    // where the chain start costs accumulator-register copies.
    constexpr bool kNegD = !kGroups || !kDrop;
    uint32_t mk[2][4][4];  // keep words of rows 32 qb + 8 g + 4 h + e (this wave's keys)
    op_t pk[2][2], sk[2][2];

    auto read = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < G_V0) {
        constexpr int qb = i / NS, t = (i % NS) / 2, isdp = i % 2;
        ring[i % RING] = rd128(oq[t] + isdp * QTB + 32 * qb * RB);
      } else {
        constexpr int j = i - G_V0, qb = j / NV, jj = j % NV;
        constexpr int t2 = jj / (2 * NDB), db = (jj / 2) % NDB, isdv = 1 - jj % 2;
        constexpr int imm = isdv * QTB + (32 * qb + 16 * t2) * RB;
        ring[i % RING] = tr_pair(lds + otr[db][0] + imm, lds + otr[db][1] + imm);
      }
    };
    auto mfma = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const op_t& x = ring[i % RING];
      if constexpr (i < G_V0) {
        constexpr int qb = i / NS, t = (i % NS) / 2;
        if constexpr (i % 2 == 0)
          s[qb] = M::mma(x, kr[t], t == 0 ? floatx16{} : s[qb]);
        else
          dp[qb] = M::mma(x, vr[t], t == 0 ? (kNegD ? nd[qb] : floatx16{}) : dp[qb]);
      } else {
        constexpr int j = i - G_V0, qb = j / NV, jj = j % NV;
        constexpr int t2 = jj / (2 * NDB), db = (jj / 2) % NDB;
        if constexpr (jj % 2 == 0)
          dv[db] = M::mma(x, pk[qb][t2], dv[db]);
        else
          dk[db] = M::mma(x, sk[qb][t2], dk[db]);
      }
    };
    // Softmax of accumulator register r of block qb in two stages one slot
    // apart (so no instruction waits on the one before it):
    //   A: P = exp2(s c - lse2), masked;   B: dS = P (dP - D) (with kNegD the
    //   accumulator already holds dP - D), and each
    //   completed pair of P and dS is rounded into the dV / dK operands.
    auto soft_a = [&](int qb, int r) {
      const int g = r >> 2, e = r & 3;
      float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c2, -lv[qb][g][e]));
      if constexpr (kMask) {
        const int rel = 32 * qb + 8 * g + e;
        p = in_range(rel, rg) ? p : 0.f;
      }
      s[qb][r] = p;
    };
    auto soft_b = [&](int qb, int r) {
      if constexpr (kDrop) {
        // keep bit of (row, this lane's key) as a mask: 0 or all ones
        uint32_t m;
        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(mk[qb][r >> 2][r & 3]), "v"(c));
        const float nd4 = dv4[qb][r >> 2][r & 3];  // -D kp
        if constexpr (kNegD) {  // the accumulator holds dP - D kp
          uint32_t sel;
          asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(sel) : "v"(m), "v"(dp[qb][r]), "v"(nd4));
          dp[qb][r] = s[qb][r] * __uint_as_float(sel);
        } else {
          dp[qb][r] = s[qb][r] * (__uint_as_float(__float_as_uint(dp[qb][r]) & m) + nd4);
        }
        s[qb][r] = __uint_as_float(__float_as_uint(s[qb][r]) & m);
      } else if constexpr (kNegD) {
        dp[qb][r] = s[qb][r] * dp[qb][r];
      } else {
        dp[qb][r] = s[qb][r] * (dp[qb][r] + dv4[qb][r >> 2][r & 3]);
      }
      if (r & 1) {
        pk[qb][r >> 3][(r & 7) - 1] = static_cast<bf16>(s[qb][r - 1]);
        pk[qb][r >> 3][r & 7] = static_cast<bf16>(s[qb][r]);
        sk[qb][r >> 3][(r & 7) - 1] = static_cast<bf16>(dp[qb][r - 1]);
        sk[qb][r >> 3][r & 7] = static_cast<bf16>(dp[qb][r]);
      }
    };
    auto valu = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      // lse2 / D of rows 8g + 4h .. 8g + 4h + 3 of block qb, two slots before
      // the softmax of its registers 4g .. 4g + 3 (short live ranges)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (m == kv_soft_slot(qb, 4 * g) - 2) {
            const int off = olr + (32 * qb + 8 * g) * 4;
            lv[qb][g] = *reinterpret_cast<const floatx4*>(reinterpret_cast<const char*>(lse_s) + off);
            if constexpr (!kNegD || kDrop)
              dv4[qb][g] = *reinterpret_cast<const floatx4*>(reinterpret_cast<const char*>(drow_s) + off);
            if constexpr (kDrop) {
              typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
              const u32x4_t m4 = *reinterpret_cast<const u32x4_t*>(
                  reinterpret_cast<const char*>(mask_s) + omk + (32 * qb + 8 * g) * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) mk[qb][g][e] = m4[e];
            }
          }
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (m == kv_soft_slot(qb, r)) soft_a(qb, r);
          if (m == kv_soft_slot(qb, r) + 1) soft_b(qb, r);
        }
      }
    };

    if constexpr (!kNext) start_copy(tile + 1, b ^ 1);
    static_assert(COPY_EVERY * (2 * Dma::PARTS - 1) + 1 < NOPS + AHEAD, "every copy has a slot");
    static_assert(COPY_EVERY * (2 * KvDma::PARTS - 1) + 3 < NOPS + AHEAD, "every K / V copy has a slot");
    static_for<NOPS + AHEAD>([&](auto sc) {
      constexpr int sl = decltype(sc)::value;
      if constexpr (sl == 0) {
        if constexpr (kNext)
          load_rows_of(nx.lse_b, nx.drow_b, nx.sq, nx.skv, nx.block, nx.dh, nx.lo, b ^ 1);
        else
          load_rows(tile + 1, b ^ 1);
      }
      // the next unit's K / V rows, one copy every COPY_EVERY slots from slot 3
      if constexpr (kNext && sl % COPY_EVERY == 3 && sl / COPY_EVERY < 2 * KvDma::PARTS)
        kv_stage_issue(std::integral_constant<int, sl / COPY_EVERY>{});
      // -D of block qb's rows, three slots before its first dP product
      // (product NS qb + 1, issued at slot NS qb + 1 + AHEAD)
      if constexpr (kNegD && (sl == AHEAD - 2 || sl == NS + AHEAD - 2)) {
        constexpr int qb = sl < NS ? 0 : 1;
        const char* base = reinterpret_cast<const char*>(drow_s) + olr + 32 * qb * 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const floatx4 f = *reinterpret_cast<const floatx4*>(base + 8 * g * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) nd[qb][4 * g + e] = f[e];
        }
      }
      // one copy instruction every COPY_EVERY slots from slot 1
      if constexpr (sl % COPY_EVERY == 1 && sl / COPY_EVERY < 2 * Dma::PARTS) {
        constexpr int pt = sl / COPY_EVERY;
        if constexpr (pt % 2 == 0)
          cp_q.template issue<pt / 2>();
        else
          cp_dy.template issue<pt / 2>();
      }
      if constexpr (sl < NOPS) read(std::integral_constant<int, sl>{});
      if constexpr (sl >= AHEAD) {
        mfma(std::integral_constant<int, sl - AHEAD>{});
        valu(std::integral_constant<int, sl - AHEAD>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto flip = [&](int b) {  // move the lane offsets to the other slab
    const int dr = b ? -SLAB : SLAB;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
      oq[t] += dr;
      asm volatile("" : "+v"(oq[t]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      otr[db][0] += dr;
      otr[db][1] += dr;
      asm volatile("" : "+v"(otr[db][0]), "+v"(otr[db][1]));
    }
    olr += b ? -(int)sizeof(lse_s[0]) : (int)sizeof(lse_s[0]);
    asm volatile("" : "+v"(olr));
    if constexpr (kDrop) {
      omk += b ? -4 * 4 * BM : 4 * 4 * BM;
      asm volatile("" : "+v"(omk));
    }
  };
  int cur = 0;  // slab of the current tile; a head or unit starts where the last one ended
  // tiles [from, to] in order, each body branch-free (masked or not)
  auto run = [&](auto mask_tag, int from, int to) __attribute__((always_inline)) {
    for (int tile = from; tile <= to; ++tile) {
      step(mask_tag, tile, cur, std::false_type{});
      if (tile < hi) store_rows(cur ^ 1);
      wait_vmem();
      __syncthreads();
      flip(cur);
      cur ^= 1;
    }
  };
  // the first query tile of head hq of the current unit into slab cur, with
  // its lse2 / -D rows (and keep bits); waited for by the caller
  auto copy_first = [&]() {
    if (lo <= hi) {
      start_copy(lo, cur);
      copy_all();
      load_rows(lo, cur);
    }
  };
  // the K / V row loads are complete (the caller waited): an empty use of
  // each register lets the compiler's wait tracking know it too, so that it
  // does not count them as outstanding (and wait for the tile copies with
  // them) in the first products of every tile
  auto settle_kv = [&]() {
    if constexpr (!kGroups) {
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) asm volatile("" : : "a"(kr[t]), "a"(vr[t]));
    }
  };

  // ---- the first unit: its K / V rows and first tile
  uint32_t iv_cur = load_unit(a.items, __builtin_amdgcn_readfirstlane(load_code(work, 0)), lane);
  uint32_t iv_n1 = 0u;
  if (n_units > 1) iv_n1 = load_unit(a.items, __builtin_amdgcn_readfirstlane(load_code(work, 1)), lane);
  int32_t code_n2 = 0;  // code of the unit after the next (loaded a unit ahead of its item)
  if (n_units > 2) code_n2 = load_code(work, 2);
  {
    const UnitInfo u0 = unit_info(iv_cur);
    set_unit(u0);
    set_head(kvh * G);
    load_kv_rows(u0);
    copy_first();
    wait_vmem();
    settle_kv();
    if (lo <= hi) store_rows(cur);
    __syncthreads();
  }

  for (int k = 0; k < n_units; ++k) {
    const bool has_nxt = k + 1 < n_units;
    // the item of unit k + 2 and the code of unit k + 3 land during this unit
    uint32_t iv_n2 = 0u;
    int32_t code_n3 = 0;
    if (k + 2 < n_units) iv_n2 = load_unit(a.items, __builtin_amdgcn_readfirstlane(code_n2), lane);
    if (k + 3 < n_units) code_n3 = load_code(work, k + 3);
    key_range();
    bool pre = false;  // the last tile prefetched the next unit
    for (int gi = 0; gi < G; ++gi) {
      if (gi > 0) {  // the next query head of the group: its first tile
        set_head(kvh * G + gi);
        copy_first();
        wait_vmem();
        if (lo <= hi) store_rows(cur);
        __syncthreads();
      }
      // the unit's last tile, when masked, prefetches the next unit (not
      // with dropout, whose extra state leaves no registers for it)
      const bool last_masked = !(flo <= fhi && fhi >= hi);
      pre = !kDrop && has_nxt && gi == G - 1 && lo <= hi && last_masked;
      const int last = pre ? hi - 1 : hi;
      if (flo <= fhi) {  // masked tiles before and after the mask-free range
        run(std::true_type{}, lo, flo - 1);
        run(std::false_type{}, flo, fhi < last ? fhi : last);
        run(std::true_type{}, fhi + 1, last);
      } else {
        run(std::true_type{}, lo, last);
      }
      if constexpr (!kDrop) {
        if (pre) {
          prefetch_select(unit_info(iv_n1), cur ^ 1);
          step(std::true_type{}, hi, cur, std::true_type{});
          wait_vmem();
          __syncthreads();
          flip(cur);
          cur ^= 1;
        }
      }
    }

    // Switch: the next unit's K / V rows (the registers of this unit's are
    // free) and first tile go out before this unit's dK = scale dK^T and dV^T
    // leave, as whole rows through two LDS slices per wave of the epilogue
    // area, so the loads' latency overlaps the stores.
    const int row0 = it.block * BN + 32 * w;  // sequence-local key of the wave's slice
    bf16* const dk_dst = static_cast<bf16*>(a.dk) + ((int64_t)it.kv_base + row0) * ldkv + kvh * D;
    bf16* const dv_dst = static_cast<bf16*>(a.dv) + ((int64_t)it.kv_base + row0) * ldkv + kvh * D;
    const int nrows = it.skv - row0;
    if (has_nxt) {
      const UnitInfo n = unit_info(iv_n1);
      if (!kDrop && pre) {
        // K / V rows from the epilogue area: each wave reads its own 32 keys'
        // rows, which are exactly the slices its dK / dV take next (LDS
        // operations of one wave stay in order, so no barrier is needed)
        const int r = 32 * w + c;
#pragma unroll
        for (int t = 0; t < DSTEPS; ++t) {
          const int off = tile_off<RB>(r, (16 * t + 8 * h) * 2);
          kr[t] = *reinterpret_cast<const op_t*>(epi + off);
          vr[t] = *reinterpret_cast<const op_t*>(epi + BN * RB + off);
        }
      } else {
        load_kv_rows(n);
      }
      set_unit(n);
      set_head(kvh * G);
      if (!pre) copy_first();
    }
    static_assert(EPI >= 2 * 4 * 32 * RB && EPI >= 2 * BN * RB, "the epilogue slices fit");
    store_rows_via_lds<NDB>(dk, a.scale, epi + w * 32 * RB, dk_dst, ldkv, nrows);
    store_rows_via_lds<NDB>(dv, 1.f, epi + (4 + w) * 32 * RB, dv_dst, ldkv, nrows);
    if (has_nxt && !pre) {
      wait_vmem();
      settle_kv();
      if (lo <= hi) store_rows(cur);
      __syncthreads();
    }
    iv_cur = iv_n1;
    iv_n1 = iv_n2;
    code_n2 = code_n3;
  }
  (void)iv_cur;
}

}  // namespace swa
