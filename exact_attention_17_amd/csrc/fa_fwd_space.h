// fa_fwd_space.h -- the compiled tile-configuration space of the forward kernel, which the
// autotuner searches (page "Flash Attention 2 Chapter6", Kernel 7: enumerate the block
// shapes B_r x B_c and the warp count, drop those that do not fit or spill, time the rest).
//
// A configuration is (B_r, B_c, wavefronts, K/V stages, schedule).  The space is
//   schedule 0 (one 32-row block per wavefront): B_r in {64, 128, 256} (2, 4, 8 wavefronts)
//       x B_c in {32, 64, 128} x stages 1..4;
//   schedule 1 (two 32-row blocks per wavefront, one wavefront per SIMD): B_r in {64, 128,
//       256} (1, 2, 4 wavefronts) x B_c in {32, 64, 128}, a 2-slot K and 3-slot V ring;
//   schedule 2 (ping-pong of two groups of four wavefronts): B_r 256 x B_c in {32, 64, 128}
//       and, at d_head 64 and 128, 96, 3-slot rings;
//   schedule 4 (three wavefronts per SIMD): B_r in {64, 128} x B_c 32 x stages 2..3;
//   schedule 5 (three-group rotation, twelve wavefronts): B_r 384 x B_c 32, 3-slot rings;
// less what does not fit one CU's 160 KB of LDS and what the compiler spills registers
// for (in_space below).  Each instantiation unit compiles one part of it for one
// (d_head, dtype).
#pragma once

#include <type_traits>

#include "fa_fwd_kernel.h"

namespace fa {

// LDS bytes of a configuration (the kernel's own count: stages (K, V) tile pairs, or for
// schedule 1 a 2-slot K ring plus a 3-slot V ring).
template <int D, int BC, int STAGES, int SCHED>
constexpr int space_lds_bytes() {
  return SCHED == 1 ? 5 * BC * D * 2 : STAGES * 2 * BC * D * 2;
}

// Left out of the space, besides LDS: configurations whose registers the compiler spills
// to scratch (hipcc's per-kernel resource report for gfx950, the same for bf16 and fp16):
//   schedule 0, d_head 128, 128-key tiles: B_r 256 (any stages) and B_r 128 with one stage;
//   schedule 1 (two 32-row blocks' scores, outputs and queries per lane): d_head 128 with 64-
//       or 128-key tiles, d_head 64 with 128-key tiles;
//   schedule 4 (168 registers), d_head 128, B_r 64 with two stages.
template <int D, int BR, int BC, int NW, int STAGES, int SCHED>
constexpr bool spills() {
  if (SCHED == 0) return D == 128 && BC == 128 && (BR == 256 || (BR == 128 && STAGES == 1));
  if (SCHED == 1) return (D == 128 && BC >= 64) || (D == 64 && BC == 128);
  if (SCHED == 4) return D == 128 && BR == 64 && STAGES == 2;
  return false;
}

template <int D, int BR, int BC, int NW, int STAGES, int SCHED>
constexpr bool in_space() {
  return space_lds_bytes<D, BC, STAGES, SCHED>() <= 160 * 1024 && !spills<D, BR, BC, NW, STAGES, SCHED>();
}

template <int B, int E, typename F>
inline void host_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    host_for<B + 1, E>(f);
  }
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16, int SCHED>
inline void add_if_in_space(AddEntryFn add) {
  if constexpr (in_space<D, BR, BC, NW, STAGES, SCHED>()) add(make_entry<D, BR, BC, NW, STAGES, F16, SCHED>());
}

// Parts (one instantiation unit each, so the build compiles them in parallel):
//   0, 1, 2: schedule 0 at B_r = 64, 128, 256;  3: schedules 1, 2 and 4.
template <int D, bool F16, int PART>
void register_part(AddEntryFn add) {
  static_assert(PART >= 0 && PART < kSpaceParts, "part");
  if constexpr (PART < 3) {
    constexpr int BR = 64 << PART, NW = BR / 32;
    host_for<0, 3>([&](auto bi) {
      constexpr int BC = 32 << decltype(bi)::value;
      host_for<1, 5>([&](auto si) { add_if_in_space<D, BR, BC, NW, decltype(si)::value, F16, 0>(add); });
    });
  } else {
    host_for<0, 3>([&](auto ri) {
      constexpr int BR = 64 << decltype(ri)::value;
      host_for<0, 3>([&](auto bi) { add_if_in_space<D, BR, 32 << decltype(bi)::value, BR / 64, 2, F16, 1>(add); });
    });
    host_for<0, 3>([&](auto bi) { add_if_in_space<D, 256, 32 << decltype(bi)::value, 8, 3, F16, 2>(add); });
    if constexpr (D >= 64) add_if_in_space<D, 256, 96, 8, 3, F16, 2>(add);  // (whole 1 KB pieces)
    host_for<0, 2>([&](auto ri) {
      constexpr int BR = 64 << decltype(ri)::value;
      host_for<2, 4>([&](auto si) { add_if_in_space<D, BR, 32, BR / 32, decltype(si)::value, F16, 4>(add); });
    });
    add_if_in_space<D, 384, 32, 12, 3, F16, 5>(add);
  }
}

}  // namespace fa
