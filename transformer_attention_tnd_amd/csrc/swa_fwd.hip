// Forward kernel: online-softmax attention over the visited key tiles of one
// block of 128 query rows of one (sequence, head).
//
// Math (FlashAttentionVarLenScore API doc, "计算公式"; PyPTO-Gym
// FlashAttentionScoreGrad article, "前向公式"): out = softmax(mask(scale Q K^T)) V,
// with softmax_max / softmax_sum saved per row.  The blockwise (online)
// softmax keeps a running max m and running sum l per row and rescales the
// output accumulator when m grows, so the full score matrix never exists.
//
// Workgroup: 4 wavefronts x 32 query rows.  Each wave keeps its Q rows in
// registers and computes the transposed score block S^T = K Q^T (keys as
// rows, its 32 queries as columns), so that a lane owns one query row: the
// row max and row sum are in-lane reductions plus one swap of lane halves.
// The probabilities P^T are rounded to the input type and reused directly
// from the accumulator registers as the B operand of O^T += V^T P^T; V is
// staged transposed in LDS with its keys at the matching slot positions.
// K (row-major) and V^T tiles are double-buffered in LDS; the next tile's
// global loads are issued before the current tile's math.

#include <hip/hip_runtime.h>

#include "swa_common.hpp"

namespace swa {

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void swa_fwd_kernel(FwdArgs a) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int BM = FWD_BM, BN = FWD_BN;
  constexpr int EPV = 16 / sizeof(T);     // elements per 16-byte vector
  constexpr int CPR = D / EPV;            // 16-byte chunks per row
  constexpr int KLD = D + EPV;            // K tile row stride (16-byte pad)
  constexpr int VLD = BN + EPV;           // V^T tile row stride
  constexpr int NDB = D / 32;             // 32-wide head-dim blocks
  constexpr int NJB = BN / 32;            // 32-key blocks per tile
  constexpr int QSTEPS = D / KSTEP;       // contraction steps over d
  constexpr int PSTEPS = 32 / KSTEP;      // contraction steps per 32 keys
  constexpr int NV = BN * CPR / 256;      // 16-byte vectors per thread per tensor
  static_assert(BM == 128 && BN == 64, "kernel assumes 4 waves x 32 rows and 64-key tiles");
  static_assert(NV >= 1 && BN * CPR % 256 == 0, "tile load mapping");

  // bf16 stages V transposed (each lane reads 8 consecutive keys); fp32 reads
  // one element per lane and step, so it keeps V row-major.
  constexpr bool kVt = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T Ks[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) T Vt[2][kVt ? D * VLD : BN * KLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.n_items;
  const Item it = a.items[L - head * a.n_items];
  const int64_t ld = (int64_t)a.num_heads * D;
  const T* qg = static_cast<const T*>(a.q) + (int64_t)it.q_base * ld + head * D;
  const T* kg = static_cast<const T*>(a.k) + (int64_t)it.kv_base * ld + head * D;
  const T* vg = static_cast<const T*>(a.v) + (int64_t)it.kv_base * ld + head * D;
  const int qrow = it.block * BM + 32 * w + c;  // this lane's query row (sequence-local)
  const int lo = it.tiles & 0xffff, hi = (it.tiles >> 16) & 0xffff;
  const int flo = it.full & 0xffff, fhi = (it.full >> 16) & 0xffff;
  const float c2 = a.scale_log2;

  // Q fragments: B operand of S^T = K Q^T, lane (column qrow) holds
  // Q[qrow][KSTEP*t + KPL*h + e].
  op_t qf[QSTEPS];
  {
    const bool ok = qrow < it.sq;
    const T* qp = qg + (int64_t)(ok ? qrow : 0) * ld;
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      qf[t] = M::load(qp + KSTEP * t + KPL * h);
      if (!ok) qf[t] = op_t{};
    }
  }

  Vec16 kreg[NV], vreg[NV];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int vi = tid + 256 * p, key = vi / CPR, ch = vi % CPR;
      const int j = tile * BN + key;
      if (j < it.skv) {
        kreg[p] = load16(kg + (int64_t)j * ld + ch * EPV);
        vreg[p] = load16(vg + (int64_t)j * ld + ch * EPV);
      } else {
        kreg[p] = zero16();
        vreg[p] = zero16();
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int vi = tid + 256 * p, key = vi / CPR, ch = vi % CPR;
      *reinterpret_cast<Vec16*>(&Ks[buf][key * KLD + ch * EPV]) = kreg[p];
      if constexpr (kVt) {
        const int pos = slot_of_row<T>(key);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int d = ch * EPV + e;
          Vt[buf][d * VLD + swz(d, pos)] = vec_elem<T>(vreg[p], e);
        }
      } else {
        *reinterpret_cast<Vec16*>(&Vt[buf][key * KLD + ch * EPV]) = vreg[p];
      }
    }
  };

  floatx16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (lo <= hi) {
    load_tile(lo);
    store_tile(0);
    __syncthreads();
    for (int tile = lo; tile <= hi; ++tile) {
      const int buf = (tile - lo) & 1;
      if (tile < hi) load_tile(tile + 1);

      // S^T block jb: rows = keys 32*jb + c_row(r, h), column = this lane's query
      floatx16 s[NJB];
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        s[jb] = floatx16{};
#pragma unroll
        for (int t = 0; t < QSTEPS; ++t) {
          const op_t ka = M::load(&Ks[buf][(32 * jb + c) * KLD + KSTEP * t + KPL * h]);
          s[jb] = M::mma(ka, qf[t], s[jb]);
        }
      }

      // scale into log2 units, mask partial tiles, running max
      const bool need_mask = tile < flo || tile > fhi;
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[jb][r] * c2;
          if (need_mask) {
            const int j = tile * BN + 32 * jb + c_row(r, h);
            if (!allowed(qrow, j, it.sq, it.skv, a.mode, a.pre, a.next)) x = -INFINITY;
          }
          s[jb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[jb][r] - m_use);
          s[jb][r] = p;
          lsum += p;
        }
      }
      l_run = l_run * alpha + lsum;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      }
      m_run = m_new;

      // O^T[db] += V^T P^T
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
        for (int t2 = 0; t2 < PSTEPS; ++t2) {
          const op_t pb = M::pack(s[jb], t2);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = 32 * db + c;
            const int pos = 32 * jb + KSTEP * t2 + KPL * h;
            op_t va;
            if constexpr (kVt)
              va = M::load(&Vt[buf][d * VLD + swz(d, pos)]);
            else
              va = M::load(&Vt[buf][row_of_slot<T>(pos) * KLD + d]);
            o[db] = M::mma(va, pb, o[db]);
          }
        }
      }

      if (tile < hi) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: normalise, store out and the statistics of this lane's row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < it.sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t tok = (int64_t)it.q_base + qrow;
    T* op = static_cast<T*>(a.out) + tok * ld + head * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = static_cast<bf16>(o[db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(op + d0) = v4;
        } else {
          floatx4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * g + e] * inv;
          *reinterpret_cast<floatx4*>(op + d0) = v4;
        }
      }
    }
    const float smax = (m_run == -INFINITY) ? -INFINITY : m_run * 0.69314718055994531f;
    const floatx4 mv = {smax, smax, smax, smax};
    const floatx4 sv = {l_tot, l_tot, l_tot, l_tot};
    const int64_t so = (tok * a.num_heads + head) * 8 + 4 * h;
    *reinterpret_cast<floatx4*>(a.smax + so) = mv;
    *reinterpret_cast<floatx4*>(a.ssum + so) = sv;
  }
}

template <typename T, int D>
static int launch_fwd_t(const FwdArgs& a, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_heads;
  hipLaunchKernelGGL((swa_fwd_kernel<T, D>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_forward(const FwdArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return head_dim == 128 ? launch_fwd_t<bf16, 128>(a, stream)
                                         : launch_fwd_t<bf16, 64>(a, stream);
  return head_dim == 128 ? launch_fwd_t<float, 128>(a, stream)
                         : launch_fwd_t<float, 64>(a, stream);
}

}  // namespace swa
