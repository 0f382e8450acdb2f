// Launch of the bf16 dK/dV kernel for grouped key/value heads (each
// workgroup runs the query heads of its group one after another).  Compiled,
// like swa_bwd_kv.hip, with the matrix-core results in ordinary vector
// registers; the instantiation with dropout is in swa_bwd_kv_gqa_drop.hip
// (with that register form it spills).

#include "swa_bwd_kv.hpp"

namespace swa {

template <bool kDrop>
static int launch_bwd_kv_grouped_t(const BwdArgs& a, int head_dim, void* stream) {
  const int64_t nwg = a.n_wg;  // persistent: one workgroup per compute unit
  if (head_dim == 128)
    hipLaunchKernelGGL((swa_bwd_kv_kernel<128, true, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((swa_bwd_kv_kernel<64, true, kDrop>), dim3((unsigned)nwg), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_bwd_kv_grouped(const BwdArgs& a, int head_dim, void* stream) {
  return a.drop.words ? launch_bwd_kv_grouped_drop(a, head_dim, stream)
                      : launch_bwd_kv_grouped_t<false>(a, head_dim, stream);
}

}  // namespace swa
