// Compiled tile configurations for bf16, d_head = 64 (the tuner's search space; page
// "Flash Attention 2 Chapter6", Kernel 7: B_r x B_c x waves, plus the K/V buffering depth
// and the instruction schedule).
#include "fa_fwd_kernel.h"

namespace fa {

void register_bf16_d64(void (*add)(const KernelEntry &)) {
  add(make_entry<64, 128, 64, 4, 2, false>());
  add(make_entry<64, 128, 32, 4, 2, false>());
  add(make_entry<64, 128, 128, 4, 2, false>());
  add(make_entry<64, 64, 64, 2, 2, false>());
  add(make_entry<64, 256, 64, 8, 2, false>());
  add(make_entry<64, 128, 64, 4, 1, false>());
  add(make_entry<64, 256, 32, 4, 2, false, 1>());
  add(make_entry<64, 256, 64, 8, 3, false, 2>());
  add(make_entry<64, 256, 32, 8, 3, false, 2>());
  add(make_entry<64, 256, 32, 8, 2, false>());
  add(make_entry<64, 256, 64, 8, 3, false>());
  add(make_entry<64, 256, 64, 8, 4, false>());
  add(make_entry<64, 256, 32, 8, 4, false>());
  add(make_entry<64, 128, 32, 4, 3, false>());
  add(make_entry<64, 128, 32, 4, 2, false, 4>());
  add(make_entry<64, 128, 32, 4, 3, false, 4>());
}

}  // namespace fa
