// Compiled tile configurations for fp16, d_head = 32 (the tuner's search space; page
// "Flash Attention 2 Chapter6", Kernel 7: B_r x B_c x waves, plus the K/V buffering depth
// and the instruction schedule).
#include "fa_fwd_kernel.h"

namespace fa {

void register_fp16_d32(void (*add)(const KernelEntry &)) {
  add(make_entry<32, 128, 64, 4, 2, true>());
  add(make_entry<32, 128, 32, 4, 2, true>());
  add(make_entry<32, 128, 128, 4, 2, true>());
  add(make_entry<32, 64, 64, 2, 2, true>());
  add(make_entry<32, 256, 64, 8, 2, true>());
  add(make_entry<32, 128, 64, 4, 1, true>());
  add(make_entry<32, 256, 32, 4, 2, true, 1>());
  add(make_entry<32, 256, 64, 8, 3, true, 2>());
  add(make_entry<32, 256, 32, 8, 3, true, 2>());
  add(make_entry<32, 256, 32, 8, 2, true>());
  add(make_entry<32, 256, 64, 8, 3, true>());
  add(make_entry<32, 256, 64, 8, 4, true>());
  add(make_entry<32, 256, 32, 8, 4, true>());
  add(make_entry<32, 128, 32, 4, 3, true>());
  add(make_entry<32, 128, 32, 4, 2, true, 4>());
  add(make_entry<32, 128, 32, 4, 3, true, 4>());
}

}  // namespace fa
