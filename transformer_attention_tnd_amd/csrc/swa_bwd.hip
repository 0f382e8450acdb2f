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
//   with c = scale * log2(e); it also zeroes the fp32 dq accumulator.
// swa_bwd_kernel: one workgroup per (block of 128 keys, head); each of its 4
//   waves owns 32 keys and keeps K, V (as matrix operands) and its dK, dV
//   accumulators in registers while it walks the query tiles of the band.
//   Scores are formed as S = Q K^T (queries as rows, the wave's keys as
//   columns), so P and dS come out of the accumulators in the operand layout
//   of dV^T += dY^T P and dK^T += Q^T dS; Q and dY are staged in LDS both
//   row-major and transposed.  dS is written to LDS and each wave forms dQ for
//   one 32-wide head-dim block over all 128 keys, added to the fp32
//   accumulator with atomics (non-deterministic summation order, as the
//   explainer section 6.1 describes for the default backward).
// swa_dq_finalize_kernel: dq = scale * dq_acc rounded to the output type.

#include <hip/hip_runtime.h>

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
  float* z = a.dq_acc + row * D + ch * EPV;
#pragma unroll
  for (int e = 0; e < EPV; e += 4) *reinterpret_cast<floatx4*>(z + e) = floatx4{0.f, 0.f, 0.f, 0.f};
  if (ch == 0) {
    a.drow[row] = acc;
    const float mx = a.smax[row * 8], sm = a.ssum[row * 8];
    a.lse2[row] = (sm > 0.f && mx > -INFINITY) ? mx * 1.4426950408889634f + log2f(sm) : INFINITY;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void swa_bwd_kernel(BwdArgs a) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KPL = M::KPL, KSTEP = M::KSTEP;
  constexpr int BN = BWD_BN, BM = BWD_BM;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int CPR = D / EPV;            // 16-byte chunks per row
  constexpr int QLD = D + EPV;            // row-major Q / dY stage stride
  constexpr int TLD = BM + EPV;           // transposed Q / dY stage stride
  constexpr int SLD = BN + EPV;           // dS stage stride
  constexpr int NDB = D / 32;             // head-dim blocks
  constexpr int QB = BM / 32;             // 32-row query blocks per tile
  constexpr int DSTEPS = D / KSTEP;       // contraction steps over d
  constexpr int QSTEPS = 32 / KSTEP;      // contraction steps per 32 query rows
  constexpr int KSTEPS = BN / KSTEP;      // contraction steps over the 128 keys
  constexpr int WPD = 4 / NDB;            // waves sharing one head-dim block in dQ
  constexpr int TASKS = QB / WPD;         // dQ output blocks per wave
  constexpr int NV = BM * CPR / 256;      // 16-byte vectors per thread per tensor
  static_assert(BN == 128 && BM == 64, "kernel assumes 4 waves x 32 keys, 64-row tiles");
  static_assert(NDB <= 4 && 4 % NDB == 0 && TASKS >= 1, "head-dim split");
  static_assert(NV >= 1 && BM * CPR % 256 == 0, "tile load mapping");

  __shared__ __attribute__((aligned(16))) T Qs[BM * QLD];
  __shared__ __attribute__((aligned(16))) T dYs[BM * QLD];
  // bf16 also stages Q and dY transposed (8 consecutive query slots per
  // lane); fp32 reads one element per lane and step from the row-major copy.
  constexpr bool kTr = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T Qt[kTr ? D * TLD : 1];
  __shared__ __attribute__((aligned(16))) T dYt[kTr ? D * TLD : 1];
  __shared__ __attribute__((aligned(16))) T dSs[BM * SLD];
  __shared__ __attribute__((aligned(16))) float lse_s[BM];
  __shared__ __attribute__((aligned(16))) float drow_s[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, c = lane & 31;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int head = L / a.n_items;
  const Item it = a.items[L - head * a.n_items];
  const int N = a.num_heads;
  const int64_t ld = (int64_t)N * D;
  const T* qg = static_cast<const T*>(a.q) + (int64_t)it.q_base * ld + head * D;
  const T* dyg = static_cast<const T*>(a.dy) + (int64_t)it.q_base * ld + head * D;
  const T* kg = static_cast<const T*>(a.k) + (int64_t)it.kv_base * ld + head * D;
  const T* vg = static_cast<const T*>(a.v) + (int64_t)it.kv_base * ld + head * D;
  const int kb0 = it.block * BN;          // first key of the block (sequence-local)
  const int kw = kb0 + 32 * w + c;        // this lane's key
  const int lo = it.tiles & 0xffff, hi = (it.tiles >> 16) & 0xffff;
  const int flo = it.full & 0xffff, fhi = (it.full >> 16) & 0xffff;
  const float c2 = a.scale_log2;

  // K, V fragments: B operands of S = Q K^T and dP = dY V^T,
  // lane (column kw) holds K[kw][KSTEP*t + KPL*h + e].
  op_t kf[DSTEPS], vf[DSTEPS];
  {
    const bool ok = kw < it.skv;
    const int64_t off = (int64_t)(ok ? kw : 0) * ld;
#pragma unroll
    for (int t = 0; t < DSTEPS; ++t) {
      kf[t] = M::load(kg + off + KSTEP * t + KPL * h);
      vf[t] = M::load(vg + off + KSTEP * t + KPL * h);
      if (!ok) {
        kf[t] = op_t{};
        vf[t] = op_t{};
      }
    }
  }
  // K^T fragments for dQ = dS K: B[k = key slot][j = d], lane (column d of
  // head-dim block wd) holds K[kb0 + KSTEP*t + KPL*h + e][32*wd + c].
  const int wd = w % NDB;
  op_t ktf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    if constexpr (KPL == 1) {
      const int key = kb0 + KSTEP * t + h;
      ktf[t] = key < it.skv ? kg[(int64_t)key * ld + 32 * wd + c] : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int key = kb0 + KSTEP * t + KPL * h + e;
        ktf[t][e] = key < it.skv ? kg[(int64_t)key * ld + 32 * wd + c] : static_cast<T>(0.f);
      }
    }
  }

  floatx16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = floatx16{};
    dv[db] = floatx16{};
  }

  Vec16 qreg[NV], yreg[NV];
  float sreg = 0.f;
  auto load_qtile = [&](int tile) {
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int vi = tid + 256 * p, row = vi / CPR, ch = vi % CPR;
      const int i = tile * BM + row;
      if (i < it.sq) {
        qreg[p] = load16(qg + (int64_t)i * ld + ch * EPV);
        yreg[p] = load16(dyg + (int64_t)i * ld + ch * EPV);
      } else {
        qreg[p] = zero16();
        yreg[p] = zero16();
      }
    }
    if (tid < 2 * BM) {
      const int row = tid & (BM - 1), i = tile * BM + row;
      const int64_t idx = ((int64_t)it.q_base + i) * N + head;
      if (tid < BM)
        sreg = i < it.sq ? a.lse2[idx] : INFINITY;
      else
        sreg = i < it.sq ? a.drow[idx] : 0.f;
    }
  };
  auto store_qtile = [&]() {
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int vi = tid + 256 * p, row = vi / CPR, ch = vi % CPR;
      *reinterpret_cast<Vec16*>(&Qs[row * QLD + ch * EPV]) = qreg[p];
      *reinterpret_cast<Vec16*>(&dYs[row * QLD + ch * EPV]) = yreg[p];
      if constexpr (kTr) {
        const int pos = slot_of_row<T>(row);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int d = ch * EPV + e;
          Qt[d * TLD + swz(d, pos)] = vec_elem<T>(qreg[p], e);
          dYt[d * TLD + swz(d, pos)] = vec_elem<T>(yreg[p], e);
        }
      }
    }
    if (tid < BM)
      lse_s[tid] = sreg;
    else if (tid < 2 * BM)
      drow_s[tid - BM] = sreg;
  };

  if (lo <= hi) {
    load_qtile(lo);
    store_qtile();
  }
  __syncthreads();
  for (int tile = lo; tile <= hi; ++tile) {
    if (tile < hi) load_qtile(tile + 1);
    const bool need_mask = tile < flo || tile > fhi;

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int t = 0; t < DSTEPS; ++t) {
        const op_t qa = M::load(&Qs[(32 * qb + c) * QLD + KSTEP * t + KPL * h]);
        s = M::mma(qa, kf[t], s);
        const op_t ya = M::load(&dYs[(32 * qb + c) * QLD + KSTEP * t + KPL * h]);
        dp = M::mma(ya, vf[t], dp);
      }
      // rows of this lane: 32*qb + c_row(r, h); P = exp2(s*c - lse2), dS = P (dP - D)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb = 32 * qb + 8 * g + 4 * h;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[rb]);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&drow_s[rb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(s[r] * c2 - l4[e]);
          if (need_mask && !allowed(tile * BM + rb + e, kw, it.sq, it.skv, a.mode, a.pre, a.next))
            p = 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]);
        }
      }
      // dV^T += dY^T P ;  dK^T += Q^T dS   (contraction over the 32 query rows)
#pragma unroll
      for (int t2 = 0; t2 < QSTEPS; ++t2) {
        const op_t pb = M::pack(s, t2);
        const op_t sb = M::pack(dp, t2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + c;
          const int slot = 32 * qb + KSTEP * t2 + KPL * h;
          op_t ya, qa;
          if constexpr (kTr) {
            ya = M::load(&dYt[d * TLD + swz(d, slot)]);
            qa = M::load(&Qt[d * TLD + swz(d, slot)]);
          } else {
            ya = M::load(&dYs[row_of_slot<T>(slot) * QLD + d]);
            qa = M::load(&Qs[row_of_slot<T>(slot) * QLD + d]);
          }
          dv[db] = M::mma(ya, pb, dv[db]);
          dk[db] = M::mma(qa, sb, dk[db]);
        }
      }
      // dS (rounded to the input type) for the dQ product
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dSs[(32 * qb + c_row(r, h)) * SLD + 32 * w + c] = static_cast<T>(dp[r]);
    }
    __syncthreads();

    // dQ[32 rows x 32 d] = dS[rows, 128 keys] K[128 keys, d-block wd]
#pragma unroll
    for (int k = 0; k < TASKS; ++k) {
      const int qb = w / NDB + k * WPD;
      floatx16 acc = floatx16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const op_t sa = M::load(&dSs[(32 * qb + c) * SLD + KSTEP * t + KPL * h]);
        acc = M::mma(sa, ktf[t], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = tile * BM + 32 * qb + c_row(r, h);
        if (i < it.sq)
          unsafeAtomicAdd(a.dq_acc + ((int64_t)it.q_base + i) * ld + head * D + 32 * wd + c, acc[r]);
      }
    }
    if (tile < hi) store_qtile();
    __syncthreads();
  }

  // epilogue: this lane's key column of dK^T / dV^T
  if (kw < it.skv) {
    const int64_t tok = (int64_t)it.kv_base + kw;
    T* dkp = static_cast<T*>(a.dk) + tok * ld + head * D;
    T* dvp = static_cast<T*>(a.dv) + tok * ld + head * D;
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

template <typename T, int D>
static int launch_bwd_t(const BwdArgs& a, void* stream) {
  const int64_t nwg = (int64_t)a.n_items * a.num_heads;
  hipLaunchKernelGGL((swa_bwd_kernel<T, D>), dim3((unsigned)nwg), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_backward(const BwdArgs& a, int dtype, int head_dim, void* stream) {
  if (dtype == 1) return head_dim == 128 ? launch_bwd_t<bf16, 128>(a, stream)
                                         : launch_bwd_t<bf16, 64>(a, stream);
  return head_dim == 128 ? launch_bwd_t<float, 128>(a, stream)
                         : launch_bwd_t<float, 64>(a, stream);
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

}  // namespace swa
