// Compiled backward kernels: 32 keys per wavefront; four wavefronts per workgroup at d_head
// 64 and 128, two at d_head 32 (so that the dQ tiles of a 64-row query step spread evenly).
// Each in two forms: dQ by atomics in the main kernel, or by a separate pass.
#include "fa_bwd_kernel.h"

namespace fa {

int bwd_block_keys(int d_head) { return d_head == 32 ? 64 : 128; }

template <bool AT>
hipError_t launch_bwd_t(const BwdArgs &a, int d_head, bool f16, hipStream_t stream) {
  switch (d_head) {
    case 32:
      return f16 ? launch_fa_bwd<32, 2, true, AT>(a, stream) : launch_fa_bwd<32, 2, false, AT>(a, stream);
    case 64:
      return f16 ? launch_fa_bwd<64, 4, true, AT>(a, stream) : launch_fa_bwd<64, 4, false, AT>(a, stream);
    case 128:
      return f16 ? launch_fa_bwd<128, 4, true, AT>(a, stream) : launch_fa_bwd<128, 4, false, AT>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdArgs &a, int d_head, int dtype, hipStream_t stream) {
  const bool f16 = dtype == 1;
  return a.dq_acc ? launch_bwd_t<true>(a, d_head, f16, stream) : launch_bwd_t<false>(a, d_head, f16, stream);
}

}  // namespace fa
