// Launch of the bf16 dK/dV kernel with one query head per key/value head.
// This file is compiled with the matrix-core results in ordinary vector
// registers (see build.py), so the softmax reads the S and dP accumulators
// without accumulator-register copies.

#include "swa_bwd_kv.hpp"

namespace swa {

template <bool kDrop>
static int launch_bwd_kv_t(const BwdArgs& a, int head_dim, void* stream) {
  const int64_t nwg = a.n_wg;  // persistent: one workgroup per compute unit
  if (head_dim == 128)
    hipLaunchKernelGGL((swa_bwd_kv_kernel<128, false, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_bwd_kv_kernel<64, false, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_kv(const BwdArgs& a, int head_dim, void* stream) {
  if (a.num_kv_heads != a.num_heads) return launch_bwd_kv_grouped(a, head_dim, stream);
  return a.drop.words ? launch_bwd_kv_t<true>(a, head_dim, stream)
                      : launch_bwd_kv_t<false>(a, head_dim, stream);
}

}  // namespace swa
