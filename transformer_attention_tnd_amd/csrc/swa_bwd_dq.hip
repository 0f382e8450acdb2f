// Backward dQ kernel (bf16): the Q-outer pass of the two-pass backward of
// the PyPTO-Gym FlashAttentionScoreGrad article (两趟循环结构); the KV-outer
// pass (dK, dV) is swa_bwd_kv_kernel.
//
// One workgroup per (block of 128 query rows, head); each of its 4 waves
// owns 32 rows, keeps its Q and dY rows in registers (B operands of
// S^T = K Q^T and dP^T = V dY^T, so that a lane owns one query row and its
// lse2 and D are per-lane scalars) and its dQ^T accumulator, and walks the
// key tiles (64 keys) of the band: P = exp2(S^T c - lse2), dS = P (dP - D),
// dQ^T += K^T dS^T with K^T from the key tile through transposing LDS reads.
// dq = scale dQ is written once, in the input type.  It runs first: its
// prologue also computes D = rowsum(dY o O) and lse2 of its rows (the
// backward preprocess) and stores them for the dK/dV kernel.  The products of a tile
// form one software pipeline (see swa_pipe.hpp); this file is compiled with
// the matrix-core results in ordinary vector registers, so the softmax
// reads them without copies.

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "swa_common.hpp"
#include "swa_pipe.hpp"

namespace swa {

template <int D, bool kDrop>
__global__ __launch_bounds__(256, 1) void swa_bwd_dq_kernel(BwdArgs a) {
  using M = Mfma<bf16>;
  using op_t = M::op_t;
  constexpr int BQ = 128;              // query rows per unit
  constexpr int BN = 64;               // keys per tile
  constexpr int RB = D * 2;            // row bytes
  constexpr int KTB = BN * RB;         // K or V tile bytes
  constexpr int SLAB = 2 * KTB;        // K | V
  constexpr int STB = BQ * RB;         // one staged [BQ, D] block (Q, dY or O)
  constexpr int NDB = D / 32;          // head-dim blocks
  constexpr int DSTEPS = D / 16;       // contraction steps over d
  // products of one tile, in issue order: S^T/dP^T of keys 0-31, of keys
  // 32-63, dQ^T from keys 0-31, from keys 32-63
  constexpr int NS = 2 * DSTEPS, NQ = 2 * NDB;
  constexpr int G_S1 = NS, G_Q0 = 2 * NS, G_Q1 = G_Q0 + NQ, NOPS = G_Q1 + NQ;
  constexpr int AHEAD = SWA_BWD_AHEAD, RING = AHEAD + 1;
  constexpr int COPY_EVERY = 4;  // pipeline slots between copy instructions
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  using Dma = TileDma<bf16, D, BN>;   // a K or V tile
  using SDma = TileDma<bf16, D, BQ>;  // a staged block
  // The next unit's Q, dY and O rows are staged at the switch, after the
  // epilogue.  (Issued during the unit's tiles they cost more than they hide:
  // vector-memory operations complete in order, so every later wait for a
  // tile copy also waited for these loads from HBM.)
  constexpr int SPARTS = 3 * SDma::PARTS;
  static_assert(COPY_EVERY * (2 * Dma::PARTS - 1) + 1 < NOPS + AHEAD, "every copy has a slot");
  // Slot of the first softmax stage of register r of key block jb (spread as
  // in the dK/dV kernel, before the dQ products that use it).
  constexpr auto dq_soft_slot = [](int jb, int r) {
    const int rel = jb == 0 ? G_S1 : G_Q0, last = (jb == 0 ? G_Q0 : G_Q1) + NDB - 2;
    return rel + (r * (last - rel)) / 15;
  };
  static_assert(dq_soft_slot(0, 7) + 1 < G_Q0 && dq_soft_slot(1, 7) + 1 < G_Q1 &&
                dq_soft_slot(0, 15) + 1 < G_Q0 + NDB && dq_soft_slot(1, 15) + 1 < G_Q1 + NDB,
                "softmax stages finish before the products that use them");

  // two slabs (K | V of tiles t and t + 1), then the staging area (Q | dY | O
  // rows of the next unit, swizzled row-major [BQ, D] blocks)
  __shared__ __attribute__((aligned(1024))) char lds[2 * SLAB + 3 * STB];
  char* const stage = lds + 2 * SLAB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int64_t ld = (int64_t)a.num_heads * D;       // q / dy / dq row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v row stride
  const float c2 = a.scale_log2;
  const int32_t* work = a.work + a.work_off[blockIdx.x];
  const int n_units = a.work_off[blockIdx.x + 1] - a.work_off[blockIdx.x];
  if (n_units <= 0) return;

  // K / V of unit u's sequence and key/value head (grouped heads share K / V)
  auto kv_off = [&](const UnitInfo& u) {
    return (int64_t)u.kv_base * ldkv + (u.head / (a.num_heads / a.num_kv_heads)) * D;
  };
  // Q / dY / O / dq rows of unit u's sequence and head
  auto q_off = [&](const UnitInfo& u) { return (int64_t)u.q_base * ld + u.head * D; };

  // ---- the current unit
  int lo = 1, hi = 0, flo = 1, fhi = 0;
  int skv = 0;                         // key length of the sequence
  const bf16* kg = nullptr;            // K / V of the unit
  const bf16* vg = nullptr;
  int qrow = 0, q_sq = 0;              // this lane's query row (sequence-local), Sq
  // B operands of S^T and dP^T: lane (column qrow) holds Q[qrow][16t + 8h + e], dY likewise
  op_t qf[DSTEPS], yf[DSTEPS];
  // this row's lse2 and D (rows past the end: P = 0); with dropout lse2 +
  // log2(kp) and D kp
  float lse = INFINITY, drow = 0.f;
  int j_min = 0, j_max = -1;         // keys allowed for this lane's row
  // dP^T chains start from -D instead of zero, so the accumulator ends as
  // dP - D and dS = P (dP - D) is one multiply.  With dropout (keep bit Z,
  // probability kp) the chains start from -D kp and P is formed as P / kp:
  // dS = P (Z dP / kp - D) = (P / kp) (Z ? dP - D kp : -D kp), a select and
  // one multiply.
  floatx16 ndrow;
  floatx16 acc[NDB];  // dQ^T: rows = head dim 32 db + c_row(r, h), column = this lane's row

  // Dropout keep bits of this lane's row for the 64 keys of a tile (three
  // 32-bit words, funnel-shifted in the softmax; bit k = key 64 t + k).  The
  // words of tile t + 1 are loaded during tile t; the wait at the end of each
  // tile covers them.
  uint32_t mw[3] = {0u, 0u, 0u}, mnext[3] = {0u, 0u, 0u};
  uint32_t msh = 0, mshnext = 0;
  int64_t drop_row = 0;
  auto load_mask = [&](int tile) {
    if constexpr (kDrop) {
      const int64_t bit = drop_row + (int64_t)tile * BN;
      const int64_t wd = bit >> 5;
      mshnext = (uint32_t)(bit & 31);
#pragma unroll
      for (int e = 0; e < 3; ++e)
        mnext[e] = (qrow < q_sq && wd + e < a.drop.n_words) ? a.drop.words[wd + e] : 0u;
    }
  };

  // Lane offsets (slab of the current tile)
  int ok_[DSTEPS];  // 128-bit read of key row c, chunk 2t + h
  int otr[NDB][2];  // transposing reads of the K tile, head-dim block db
#pragma unroll
  for (int t = 0; t < DSTEPS; ++t) ok_[t] = tile_off<RB>(c, (16 * t + 8 * h) * 2);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_offsets<RB>(lane, db, otr[db][0], otr[db][1]);

  // copies of a key tile's K and V into a slab, issued part by part from the
  // pipeline of the tile before; nvalid = 0 copies zeros (no memory read)
  Dma cp_k, cp_v;
  auto start_copy = [&](const bf16* k0, const bf16* v0, int nvalid, int tile, int b) {
    char* slab = lds + b * SLAB;
    cp_k.init(k0 + (int64_t)tile * BN * ldkv, ldkv, nvalid, slab, tid);
    cp_v.init(v0 + (int64_t)tile * BN * ldkv, ldkv, nvalid, slab + KTB, tid);
  };
  auto copy_tile_all = [&]() {
    static_for<Dma::PARTS>([&](auto pc) {
      cp_k.template issue<decltype(pc)::value>();
      cp_v.template issue<decltype(pc)::value>();
    });
  };
  // the first key tile of unit u into slab b (if it has one); returns whether copied
  auto copy_first_tile = [&](const UnitInfo& u, int b, bool burst) {
    const int ulo = u.tiles0 & 0xffff, uhi = (u.tiles0 >> 16) & 0xffff;
    if (ulo > uhi) return false;
    const int64_t ko = kv_off(u);
    start_copy(static_cast<const bf16*>(a.k) + ko, static_cast<const bf16*>(a.v) + ko,
               u.skv - ulo * BN, ulo, b);
    if (burst) copy_tile_all();
    return true;
  };

  // Staging copies of a unit's Q, dY and O blocks.  The three blocks share
  // the lane offsets (the source rows are ld elements apart in each tensor);
  // part p is part p % PARTS of block p / PARTS.
  SDma st;
  st.init(static_cast<const bf16*>(a.q), ld, 0, stage, tid);  // lane offsets, step, destination
  u32x4 srs[3];  // sources of the staged blocks
  auto stage_select = [&](const UnitInfo& u) {
    const int nv = u.sq - u.block * BQ;
    const uint32_t nrec = nv <= 0 ? 0u : (uint32_t)((nv < BQ ? nv : BQ) - 1) * (uint32_t)(ld * 2) + RB;
    const int64_t off = q_off(u) + (int64_t)u.block * BQ * ld;
    srs[0] = buffer_rsrc(static_cast<const bf16*>(a.q) + off, nrec);
    srs[1] = buffer_rsrc(static_cast<const bf16*>(a.dy) + off, nrec);
    srs[2] = buffer_rsrc(static_cast<const bf16*>(a.out) + off, nrec);
  };
  auto stage_issue = [&](auto pc) {
    constexpr int p = decltype(pc)::value, blk = p / SDma::PARTS, pt = p % SDma::PARTS;
    dma16_so(srs[blk], st.voff, pt * st.vstep, st.dst + blk * STB + pt * 256 * 16);
  };
  auto stage_all = [&](const UnitInfo& u) {
    stage_select(u);
    static_for<SPARTS>([&](auto pc) { stage_issue(pc); });
  };
  // statistics of this lane's row of unit u (softmax_max, softmax_sum; column 0)
  auto load_stats = [&](const UnitInfo& u, float& m, float& sm) {
    const int r = u.block * BQ + 32 * w + c;
    const int64_t so = (((int64_t)u.q_base + (r < u.sq ? r : 0)) * a.num_heads + u.head) * 8;
    m = a.smax[so];
    sm = a.ssum[so];
  };

  // Switch to unit u: its Q, dY, O rows from the staging area, its row
  // terms D and lse2 (the backward preprocess: D = rowsum(dY o O) with fp32
  // products, this lane's half of the row plus the other half from lane l ^ 32,
  // which holds the same row) stored for the dK/dV kernel, and its key range.
  auto switch_in = [&](const UnitInfo& u, float smx, float ssm) {
    lo = u.tiles0 & 0xffff;
    hi = (u.tiles0 >> 16) & 0xffff;
    flo = u.full0 & 0xffff;
    fhi = (u.full0 >> 16) & 0xffff;
    skv = u.skv;
    q_sq = u.sq;
    kg = static_cast<const bf16*>(a.k) + kv_off(u);
    vg = static_cast<const bf16*>(a.v) + kv_off(u);
    qrow = u.block * BQ + 32 * w + c;
    const bool row_ok = qrow < u.sq;
    op_t of[DSTEPS];
    {
      // (rows past the sequence were staged as zeros; the selects also keep
      // the compiler from tying these registers to the loads, which cost
      // accumulator-register copies in every tile)
      const int r = 32 * w + c;
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        const int off = tile_off<RB>(r, (16 * t + 8 * h) * 2);
        qf[t] = row_ok ? *reinterpret_cast<const op_t*>(stage + off) : op_t{};
        yf[t] = row_ok ? *reinterpret_cast<const op_t*>(stage + STB + off) : op_t{};
        of[t] = row_ok ? *reinterpret_cast<const op_t*>(stage + 2 * STB + off) : op_t{};
      }
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float dp4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 y2 = {yf[t][2 * e], yf[t][2 * e + 1]}, o2 = {of[t][2 * e], of[t][2 * e + 1]};
        dp4[e] = __builtin_amdgcn_fdot2_f32_bf16(y2, o2, dp4[e], false);
      }
    }
    const float dpart = (dp4[0] + dp4[1]) + (dp4[2] + dp4[3]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart), __float_as_uint(dpart),
                                                     false, false);
    lse = INFINITY;
    drow = 0.f;
    if (row_ok) {
      drow = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      lse = (ssm > 0.f && smx > -INFINITY) ? smx * 1.4426950408889634f + log2f(ssm) : INFINITY;
      if constexpr (kDrop) {
        drow *= 1.f / a.drop.rkp;
        lse += a.drop.log2kp;
      }
      if (h == 0) {
        const int64_t at = (int64_t)u.head * a.t_q + u.q_base + qrow;
        a.drow[at] = -drow;  // the dK/dV kernel starts its dP chains from it
        a.lse2[at] = lse;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ndrow[r] = -drow;
    j_min = 0;
    j_max = u.skv - 1;
    if (a.mode != 0) {  // 64-bit: pre / next may be near the int range
      const int64_t lo64 = (int64_t)qrow - u.pre, hi64 = (int64_t)qrow + u.next;
      j_min = lo64 < 0 ? 0 : (lo64 > u.skv ? u.skv : (int)lo64);
      j_max = hi64 < j_max ? (hi64 < -1 ? -1 : (int)hi64) : j_max;
    }
    if (!row_ok) j_max = -1;
    if constexpr (kDrop)
      drop_row = u.drop_base + (int64_t)u.head * u.sq * u.skv + (int64_t)(row_ok ? qrow : 0) * u.skv;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
  };

  // ---- the units after the current one: unit k + 1 (iv_n1), k + 2 (iv_n2,
  // loaded while unit k runs) and the code of unit k + 3
  uint32_t iv_n1 = 0u;
  bool has_nxt = false;
  bool first_copied = false;  // the next unit's first tile is in its slab

  auto rd128 = [&](int off) { return *reinterpret_cast<const op_t*>(lds + off); };

  // One key tile (slab b): S^T, dP^T, P, dS, dQ^T += K^T dS^T; also issues
  // the copies of the tile after it into slab b ^ 1 (the next key tile of
  // this unit, or the first of the next unit).
  auto step = [&](auto mask_tag, int tile, int b) {
    constexpr bool kMask = decltype(mask_tag)::value;
    // key 32 jb + 8 g + 4 h + e of the tile is allowed iff 32 jb + 8 g + e lies in the lane's range rg
    LaneRange rg{0, 0u};
    if constexpr (kMask) rg = lane_range(j_min - tile * BN - 4 * h, j_max - tile * BN - 4 * h, BN);
    op_t ring[RING];
    floatx16 s[2], dp[2];
    op_t sk[2][2];
    // keep bits of this lane's keys: block jb, register r -> key 32 jb + c_row(r, h)
    uint32_t keep[2] = {0u, 0u};
    if constexpr (kDrop) {
      keep[0] = __builtin_amdgcn_alignbit(mw[1], mw[0], msh) >> (4 * h);
      keep[1] = __builtin_amdgcn_alignbit(mw[2], mw[1], msh) >> (4 * h);
    }

    auto read = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < G_Q0) {
        constexpr int jb = i / NS, t = (i % NS) / 2, isv = i % 2;
        ring[i % RING] = rd128(ok_[t] + isv * KTB + 32 * jb * RB);
      } else {
        constexpr int j = i - G_Q0, jb = j / NQ, t2 = (j % NQ) / NDB, db = j % NDB;
        constexpr int imm = (32 * jb + 16 * t2) * RB;
        ring[i % RING] = tr_pair(lds + otr[db][0] + imm, lds + otr[db][1] + imm);
      }
    };
    auto mfma = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const op_t& x = ring[i % RING];
      if constexpr (i < G_Q0) {
        constexpr int jb = i / NS, t = (i % NS) / 2;
        if constexpr (i % 2 == 0)
          s[jb] = M::mma(x, qf[t], t == 0 ? floatx16{} : s[jb]);
        else
          dp[jb] = M::mma(x, yf[t], t == 0 ? ndrow : dp[jb]);  // ndrow: -D (with dropout -D kp)
      } else {
        constexpr int j = i - G_Q0, jb = j / NQ, t2 = (j % NQ) / NDB, db = j % NDB;
        acc[db] = M::mma(x, sk[jb][t2], acc[db]);
      }
    };
    // Softmax of accumulator register r of key block jb in two stages one
    // slot apart: A: P = exp2(s c - lse2), masked;  B: dS = P (dP - D) (the
    // accumulator already holds dP - D), and
    // each completed pair of dS is rounded into the operand of dQ^T.
    auto soft_a = [&](int jb, int r) {
      float p = __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -lse));
      if constexpr (kMask) {
        const int rel = 32 * jb + 8 * (r >> 2) + (r & 3);
        p = in_range(rel, rg) ? p : 0.f;
      }
      s[jb][r] = p;
    };
    auto soft_b = [&](int jb, int r) {
      if constexpr (kDrop) {
        // keep bit as a mask (signed one-bit field extract: 0 or all ones),
        // then (P / kp) (Z ? dP - D kp : -D kp)
        uint32_t m, sel;
        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(keep[jb]), "n"(8 * (r >> 2) + (r & 3)));
        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(sel) : "v"(m), "v"(dp[jb][r]), "v"(-drow));
        dp[jb][r] = s[jb][r] * __uint_as_float(sel);
      } else {
        dp[jb][r] = s[jb][r] * dp[jb][r];
      }
      if (r & 1) {
        sk[jb][r >> 3][(r & 7) - 1] = static_cast<bf16>(dp[jb][r - 1]);
        sk[jb][r >> 3][r & 7] = static_cast<bf16>(dp[jb][r]);
      }
    };
    auto valu = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (m == dq_soft_slot(jb, r)) soft_a(jb, r);
          if (m == dq_soft_slot(jb, r) + 1) soft_b(jb, r);
        }
      }
    };

    if (tile < hi) {
      start_copy(kg, vg, skv - (tile + 1) * BN, tile + 1, b ^ 1);
    } else if (!(has_nxt && (first_copied = copy_first_tile(unit_info(iv_n1), b ^ 1, false)))) {
      start_copy(kg, vg, 0, tile + 1, b ^ 1);  // past the range: zeros
    }
    static_for<NOPS + AHEAD>([&](auto sc) {
      constexpr int sl = decltype(sc)::value;
      // one copy instruction every COPY_EVERY slots from slot 1: the next
      // tile's K and V parts, then the staging copies
      if constexpr (sl % COPY_EVERY == 1 && sl / COPY_EVERY < 2 * Dma::PARTS) {
        constexpr int pt = sl / COPY_EVERY;
        if constexpr (pt % 2 == 0)
          cp_k.template issue<pt / 2>();
        else
          cp_v.template issue<pt / 2>();
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
      ok_[t] += dr;
      asm volatile("" : "+v"(ok_[t]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      otr[db][0] += dr;
      otr[db][1] += dr;
      asm volatile("" : "+v"(otr[db][0]), "+v"(otr[db][1]));
    }
  };
  int b = 0;  // slab of the current tile
  auto run = [&](auto mask_tag, int from, int to) {
    for (int tile = from; tile <= to; ++tile) {
      if constexpr (kDrop) {  // this tile's keep words; fetch the next tile's
#pragma unroll
        for (int e = 0; e < 3; ++e) mw[e] = mnext[e];
        msh = mshnext;
        if (tile < hi) load_mask(tile + 1);
      }
      step(mask_tag, tile, b);
      wait_vmem();  // the next tile has landed
      __syncthreads();
      flip(b);
      b ^= 1;
    }
  };

  // ---- the first unit: its rows, statistics and first tile, loaded before
  // the loop; the items of the next two units
  uint32_t iv_cur, iv_n2 = 0u;
  int32_t code_n2 = 0;
  float st_m, st_s;  // statistics of the unit switched in next
  iv_cur = load_unit(a.items, __builtin_amdgcn_readfirstlane(load_code(work, 0)), lane);
  if (n_units > 1) iv_n1 = load_unit(a.items, __builtin_amdgcn_readfirstlane(load_code(work, 1)), lane);
  if (n_units > 2) code_n2 = load_code(work, 2);
  {
    const UnitInfo u0 = unit_info(iv_cur);
    stage_all(u0);
    load_stats(u0, st_m, st_s);
    copy_first_tile(u0, 0, true);
    wait_vmem();
    __syncthreads();
  }

  for (int k = 0; k < n_units; ++k) {
    has_nxt = k + 1 < n_units;
    // the item of unit k + 2 and the code of unit k + 3 land during this unit
    int32_t code_n3 = 0;
    if (k + 2 < n_units) iv_n2 = load_unit(a.items, __builtin_amdgcn_readfirstlane(code_n2), lane);
    if (k + 3 < n_units) code_n3 = load_code(work, k + 3);
    switch_in(unit_info(iv_cur), st_m, st_s);
    if constexpr (kDrop) {
      if (lo <= hi) load_mask(lo);
    }
    __syncthreads();  // every wave has read the staging area
    float nm = 0.f, ns = 0.f;
    first_copied = false;
    if (has_nxt) load_stats(unit_info(iv_n1), nm, ns);
    if (flo <= fhi) {  // masked tiles before and after the mask-free range
      run(std::true_type{}, lo, flo - 1);
      run(std::false_type{}, flo, fhi);
      run(std::true_type{}, fhi + 1, hi);
    } else {
      run(std::true_type{}, lo, hi);
    }

    // dq = scale dQ (zero for a row that attends no key), as whole rows
    // through the wave's own LDS slice of the free slab (the last tile's)
    static_assert(4 * 32 * RB <= SLAB, "the staging slices fit in a slab");
    {
      const UnitInfo u = unit_info(iv_cur);
      const int row0 = u.block * BQ + 32 * w;  // sequence-local row of the wave's slice
      store_rows_via_lds<NDB>(acc, a.scale, lds + (b ^ 1) * SLAB + w * 32 * RB,
                              static_cast<bf16*>(a.dq) + q_off(u) + (int64_t)row0 * ld, ld,
                              u.sq - row0);
    }
    __syncthreads();
    if (has_nxt) {
      // the next unit's rows (and its first tile, if the last tile of this
      // unit could not copy it)
      const UnitInfo n = unit_info(iv_n1);
      stage_all(n);
      if (!first_copied) copy_first_tile(n, b, true);
      wait_vmem();
      __syncthreads();
    }
    st_m = nm;
    st_s = ns;
    iv_cur = iv_n1;
    iv_n1 = iv_n2;
    code_n2 = code_n3;
  }
}

template <bool kDrop>
static int launch_dq_t(const BwdArgs& a, int head_dim, void* stream) {
  const int64_t nwg = a.n_wg;  // persistent: one workgroup per compute unit
  if (head_dim == 128)
    hipLaunchKernelGGL((swa_bwd_dq_kernel<128, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_bwd_dq_kernel<64, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_dq(const BwdArgs& a, int head_dim, void* stream) {
  return a.drop.words ? launch_dq_t<true>(a, head_dim, stream)
                      : launch_dq_t<false>(a, head_dim, stream);
}

}  // namespace swa
