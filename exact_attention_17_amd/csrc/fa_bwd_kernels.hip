// Compiled backward kernels: 32 keys per wavefront; four wavefronts per workgroup at d_head
// 64 and 128, two at d_head 32 (so that the dQ tiles of a 64-row query step spread evenly).
#include "fa_bwd_kernel.h"

namespace fa {

int bwd_block_keys(int d_head) { return d_head == 32 ? 64 : 128; }

hipError_t launch_bwd(const BwdArgs &a, int d_head, int dtype, hipStream_t stream) {
  const bool f16 = dtype == 1;
  switch (d_head) {
    case 32:
      return f16 ? launch_fa_bwd<32, 2, true>(a, stream) : launch_fa_bwd<32, 2, false>(a, stream);
    case 64:
      return f16 ? launch_fa_bwd<64, 4, true>(a, stream) : launch_fa_bwd<64, 4, false>(a, stream);
    case 128:
      return f16 ? launch_fa_bwd<128, 4, true>(a, stream) : launch_fa_bwd<128, 4, false>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
