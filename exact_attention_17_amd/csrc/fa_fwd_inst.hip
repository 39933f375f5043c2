// fa_fwd_inst.hip -- one part of the forward kernel's compiled configuration space, for one
// (d_head, dtype).  The build compiles this file once per combination, selecting it with
// FA_INST_D (32, 64, 128), FA_INST_F16 (0 = bf16, 1 = fp16) and FA_INST_PART
// (0 .. kSpaceParts - 1; see fa_fwd_space.h), so that the parts compile in parallel.
#include "fa_fwd_space.h"

#if !defined(FA_INST_D) || !defined(FA_INST_F16) || !defined(FA_INST_PART)
#error "fa_fwd_inst.hip is compiled with -DFA_INST_D=.. -DFA_INST_F16=.. -DFA_INST_PART=.."
#endif

namespace fa {
template void register_part<FA_INST_D, FA_INST_F16 != 0, FA_INST_PART>(AddEntryFn);
}  // namespace fa
