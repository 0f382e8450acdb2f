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
  constexpr int BQ = 128;              // query rows per workgroup
  constexpr int BN = 64;               // keys per tile
  constexpr int RB = D * 2;            // row bytes
  constexpr int KTB = BN * RB;         // K or V tile bytes
  constexpr int SLAB = 2 * KTB;        // K | V
  constexpr int NDB = D / 32;          // head-dim blocks
  constexpr int DSTEPS = D / 16;       // contraction steps over d
  // products of one tile, in issue order: S^T/dP^T of keys 0-31, of keys
  // 32-63, dQ^T from keys 0-31, from keys 32-63
  constexpr int NS = 2 * DSTEPS, NQ = 2 * NDB;
  constexpr int G_S1 = NS, G_Q0 = 2 * NS, G_Q1 = G_Q0 + NQ, NOPS = G_Q1 + NQ;
  constexpr int AHEAD = SWA_BWD_AHEAD, RING = AHEAD + 1;
  constexpr int COPY_EVERY = 4;  // pipeline slots between copy instructions
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  // Slot of the first softmax stage of register r of key block jb (spread as
  // in the dK/dV kernel, before the dQ products that use it).
  constexpr auto dq_soft_slot = [](int jb, int r) {
    const int rel = jb == 0 ? G_S1 : G_Q0, last = (jb == 0 ? G_Q0 : G_Q1) + NDB - 2;
    return rel + (r * (last - rel)) / 15;
  };
  static_assert(dq_soft_slot(0, 7) + 1 < G_Q0 && dq_soft_slot(1, 7) + 1 < G_Q1 &&
                dq_soft_slot(0, 15) + 1 < G_Q0 + NDB && dq_soft_slot(1, 15) + 1 < G_Q1 + NDB,
                "softmax stages finish before the products that use them");

  __shared__ __attribute__((aligned(1024))) char lds[2 * SLAB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.n_items;
  const Item it = a.items[L - head * a.n_items];
  const int64_t ld = (int64_t)a.num_heads * D;       // q / dy / dq row stride
  const int64_t ldkv = (int64_t)a.num_kv_heads * D;  // k / v row stride
  const int kvh = head / (a.num_heads / a.num_kv_heads);  // grouped heads share K / V
  const bf16* qg = static_cast<const bf16*>(a.q) + (int64_t)it.q_base * ld + head * D;
  const bf16* dyg = static_cast<const bf16*>(a.dy) + (int64_t)it.q_base * ld + head * D;
  const bf16* kg = static_cast<const bf16*>(a.k) + (int64_t)it.kv_base * ldkv + kvh * D;
  const bf16* vg = static_cast<const bf16*>(a.v) + (int64_t)it.kv_base * ldkv + kvh * D;
  const int qrow = it.block * BQ + 32 * w + c;  // this lane's query row (sequence-local)
  const int lo = it.tiles[0] & 0xffff, hi = (it.tiles[0] >> 16) & 0xffff;
  const int flo = it.full[0] & 0xffff, fhi = (it.full[0] >> 16) & 0xffff;
  const float c2 = a.scale_log2;

  // B operands of S^T and dP^T: lane (column qrow) holds Q[qrow][16t + 8h + e], dY likewise;
  // O likewise, and the row's statistics, for D and lse2 (row_stats)
  op_t qf[DSTEPS], yf[DSTEPS], of[DSTEPS];
  float lse = INFINITY, drow = 0.f;  // this row's lse2 and D (rows past the end: P = 0)
  float smx, ssm;
  const bool row_ok = qrow < it.sq;
  {
    const int64_t row = (int64_t)(row_ok ? qrow : 0);
    const int64_t off = row * ld + 8 * h;
    const bf16* og = static_cast<const bf16*>(a.out) + (int64_t)it.q_base * ld + head * D;
    const int64_t so = (((int64_t)it.q_base + row) * a.num_heads + head) * 8;
    smx = a.smax[so];
    ssm = a.ssum[so];
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
      qf[t] = row_ok ? M::load(qg + off + 16 * t) : op_t{};
      yf[t] = row_ok ? M::load(dyg + off + 16 * t) : op_t{};
      of[t] = row_ok ? M::load(og + off + 16 * t) : op_t{};
    }
  }
  // Keys allowed for this lane's row: j in [j_min, j_max] (empty past the end)
  int j_min = 0, j_max = it.skv - 1;
  if (a.mode != 0) {  // 64-bit: pre / next may be near the int range
    const int64_t lo64 = (int64_t)qrow - it.band[0], hi64 = (int64_t)qrow + it.band[1];
    j_min = lo64 < 0 ? 0 : (lo64 > it.skv ? it.skv : (int)lo64);
    j_max = hi64 < j_max ? (hi64 < -1 ? -1 : (int)hi64) : j_max;
  }
  if (qrow >= it.sq) j_max = -1;

  // dP^T chains start from -D instead of zero, so the accumulator ends as
  // dP - D and dS = P (dP - D) is one multiply (with dropout, dS = P (Z dP / kp
  // - D) needs dP alone: the chains start from zero)
  floatx16 ndrow;
  // D = rowsum(dY o O) (fp32 products; this lane's half of the row plus the
  // other half from lane l ^ 32, which holds the same row) and lse2 of this
  // lane's row, stored for the dK/dV kernel (the backward preprocess)
  auto row_stats = [&]() {
    // two bf16 products per instruction (exact in fp32) added in fp32, four chains
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
    if (row_ok) {
      drow = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      lse = (ssm > 0.f && smx > -INFINITY) ? smx * 1.4426950408889634f + log2f(ssm) : INFINITY;
      if (h == 0) {
        const int64_t at = (int64_t)head * a.t_q + it.q_base + qrow;
        a.drow[at] = -drow;  // the dK/dV kernel starts its dP chains from -D
        a.lse2[at] = lse;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ndrow[r] = kDrop ? 0.f : -drow;
  };

  // Dropout keep bits of this lane's row for the 64 keys of a tile (three
  // 32-bit words, funnel-shifted in the softmax; bit k = key 64 t + k).  The
  // words of tile t + 1 are loaded during tile t; the wait at the end of each
  // tile covers them.
  uint32_t mw[3] = {0u, 0u, 0u}, mnext[3] = {0u, 0u, 0u};
  uint32_t msh = 0, mshnext = 0;
  const int64_t drop_row = kDrop ? it.drop_base + (int64_t)head * it.sq * it.skv +
                                       (int64_t)(qrow < it.sq ? qrow : 0) * it.skv
                                 : 0;
  auto load_mask = [&](int tile) {
    if constexpr (kDrop) {
      const int64_t bit = drop_row + (int64_t)tile * BN;
      const int64_t w = bit >> 5;
      mshnext = (uint32_t)(bit & 31);
#pragma unroll
      for (int e = 0; e < 3; ++e)
        mnext[e] = (qrow < it.sq && w + e < a.drop.n_words) ? a.drop.words[w + e] : 0u;
    }
  };

  floatx16 acc[NDB];  // dQ^T: rows = head dim 32 db + c_row(r, h), column = this lane's row
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};

  // Lane offsets (slab of the current tile)
  int ok_[DSTEPS];  // 128-bit read of key row c, chunk 2t + h
  int otr[NDB][2];  // transposing reads of the K tile, head-dim block db
#pragma unroll
  for (int t = 0; t < DSTEPS; ++t) ok_[t] = tile_off<RB>(c, (16 * t + 8 * h) * 2);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_offsets<RB>(lane, db, otr[db][0], otr[db][1]);

  // copies of the next tile's K and V into its slab, issued part by part from
  // the pipeline of the current tile; a tile past the band copies zeros (no
  // memory read) into the free slab
  using Dma = TileDma<bf16, D, BN>;
  Dma cp_k, cp_v;
  auto start_copy = [&](int tile, int b) {
    const int nvalid = tile <= hi ? it.skv - tile * BN : 0;
    char* slab = lds + b * SLAB;
    cp_k.init(kg + (int64_t)tile * BN * ldkv, ldkv, nvalid, slab, tid);
    cp_v.init(vg + (int64_t)tile * BN * ldkv, ldkv, nvalid, slab + KTB, tid);
  };
  auto rd128 = [&](int off) { return *reinterpret_cast<const op_t*>(lds + off); };

  // One key tile (slab b): S^T, dP^T, P, dS, dQ^T += K^T dS^T; also issues
  // the copies of tile + 1 into slab b ^ 1.
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
          dp[jb] = M::mma(x, yf[t], t == 0 ? ndrow : dp[jb]);  // ndrow: -D (no dropout) or 0
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
        const bool kept = (keep[jb] >> (8 * (r >> 2) + (r & 3))) & 1u;
        dp[jb][r] = s[jb][r] * ((kept ? dp[jb][r] * a.drop.rkp : 0.f) - drow);
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

    start_copy(tile + 1, b ^ 1);
    static_assert(COPY_EVERY * (2 * Dma::PARTS - 1) + 1 < NOPS + AHEAD, "every copy has a slot");
    static_for<NOPS + AHEAD>([&](auto sc) {
      constexpr int sl = decltype(sc)::value;
      // one copy instruction every COPY_EVERY slots from slot 1
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

  // the first tile's copies go out before the row statistics wait for their loads
  if (lo <= hi) {
    start_copy(lo, 0);
    static_for<Dma::PARTS>([&](auto pc) {
      cp_k.template issue<decltype(pc)::value>();
      cp_v.template issue<decltype(pc)::value>();
    });
    load_mask(lo);
  }
  row_stats();
  if (lo <= hi) {
    wait_vmem();
    __syncthreads();
  }
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
  auto run = [&](auto mask_tag, int from, int to) {
    for (int tile = from; tile <= to; ++tile) {
      const int b = (tile - lo) & 1;
      if constexpr (kDrop) {  // this tile's keep words; fetch the next tile's
#pragma unroll
        for (int e = 0; e < 3; ++e) mw[e] = mnext[e];
        msh = mshnext;
        if (tile < hi) load_mask(tile + 1);
      }
      step(mask_tag, tile, b);
      wait_vmem();
      __syncthreads();
      flip(b);
    }
  };
  if (flo <= fhi) {  // masked tiles before and after the mask-free range
    run(std::true_type{}, lo, flo - 1);
    run(std::false_type{}, flo, fhi);
    run(std::true_type{}, fhi + 1, hi);
  } else {
    run(std::true_type{}, lo, hi);
  }

  // dq = scale dQ (zero for a row that attends no key), as whole rows
  // through the wave's own LDS slice (the slabs are free: every copy has
  // landed and the last tile is done)
  static_assert(4 * 32 * RB <= 2 * SLAB, "the staging slices fit in the slabs");
  __syncthreads();
  {
    const int row0 = it.block * BQ + 32 * w;  // sequence-local row of the wave's slice
    store_rows_via_lds<NDB>(acc, a.scale, lds + w * 32 * RB,
                            static_cast<bf16*>(a.dq) + ((int64_t)it.q_base + row0) * ld + head * D, ld,
                            it.sq - row0);
  }
}

template <bool kDrop>
static int launch_dq_t(const BwdArgs& a, int head_dim, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_heads;
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
