// Launch of the bf16 dK/dV kernel for grouped key/value heads with dropout.
// Compiled with the default register assignment (with the matrix-core
// results in ordinary vector registers this instantiation spills).

#include "swa_bwd_kv.hpp"

namespace swa {

int launch_bwd_kv_grouped_drop(const BwdArgs& a, int head_dim, void* stream) {
  const int64_t nwg = a.n_wg;  // persistent: one workgroup per compute unit
  if (head_dim == 128)
    hipLaunchKernelGGL((swa_bwd_kv_kernel<128, true, true>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_bwd_kv_kernel<64, true, true>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace swa
