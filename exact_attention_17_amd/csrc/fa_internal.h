// fa_internal.h -- types shared between the kernel instantiation units and the
// host library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Division by a divisor fixed for the whole launch, as a multiply-high, an add and a shift
// (division by invariant integers using multiplication, after Granlund and Montgomery): with
// shift = ceil(log2 d) and mul = floor(2^32 (2^shift - d) / d) + 1, n / d equals
// (mulhi(n, mul) + n) >> shift for every 0 <= n < 2^32; for n < 2^31 the sum cannot overflow
// 32 bits.  It replaces the kernels' work-item decoding by integer division, which the
// compiler expands to a few dozen scalar instructions per division.
struct FastDiv {
  uint32_t d;
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  const uint32_t shift = d <= 1 ? 0 : 32 - (uint32_t)__builtin_clz(d - 1);  // ceil(log2 d)
  const uint64_t mul = ((uint64_t(1) << 32) * ((uint64_t(1) << shift) - d)) / d + 1;
  return FastDiv{d, (uint32_t)mul, shift};
}

// n / f.d for 0 <= n < 2^31.
// (The high half of the 64-bit product compiles to one multiply-high instruction.)
__host__ __device__ inline uint32_t fast_div(uint32_t n, const FastDiv &f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (hi + n) >> f.shift;
}

// Kernel arguments, passed by value.
struct FaArgs {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;  // device; nullptr = dense layout
  int batch;
  int seqlen_q;  // dense: Nq; varlen: max sequence length (also the LSE row pitch)
  int seqlen_k;  // dense: Nk; varlen: max sequence length
  int heads;
  int heads_kv;  // K/V heads; query head h reads K/V head h / group
  int group;     // heads / heads_kv
  int causal;    // nonzero: key j is masked for query i when j > i
  int num_splits;  // key tiles of each query tile are divided among this many workgroups
  int n_qtiles;    // ceil(seqlen_q / br)
  int total_wgs;   // batch * heads * n_qtiles * num_splits
  // the divisors of the work-item decoding
  FastDiv div_splits, div_qtiles, div_group, div_heads_kv, div_batch;
  float scale_log2;  // scale * log2(e): scores go through exp2
  // num_splits > 1: each workgroup writes its split's normalised fp32 output and natural-log
  // LSE here instead of o / lse; the merge kernel combines them.
  float *o_part;    // [num_splits, batch, heads, seqlen_q, D]
  float *lse_part;  // [num_splits, batch, heads, seqlen_q]
};

// Arguments of the split merge kernel.
struct MergeArgs {
  const float *o_part;
  const float *lse_part;
  void *o;
  float *lse;
  const int32_t *cu_seqlens;
  int batch, seqlen_q, heads, num_splits;
};

typedef hipError_t (*LaunchFn)(const FaArgs &, hipStream_t);

// Launch the merge of num_splits partial results (defined in fa_merge.hip).
hipError_t launch_merge(const MergeArgs &a, int d_head, int dtype, hipStream_t stream);

// One compiled kernel configuration.
struct KernelEntry {
  int dtype;  // 0 bf16, 1 fp16
  int d_head;
  int br, bc, waves, stages, schedule;
  LaunchFn launch;
  const void *kernel;  // for hipFuncGetAttributes
};

typedef void (*AddEntryFn)(const KernelEntry &);

// Host-side helpers of the C ABI (fa_fwd_api.cpp) for entry points defined in other units.
// fwd_check_args: fa_fwd_ext's synchronous argument checks (no HIP call); FA_OK or an
// fa_status_t with the thread's last-error message set.  set_error: set that message and
// return status.
int fwd_check_args(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
                   int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale, int causal,
                   const int32_t *cu_seqlens, int dtype);
int set_error(int status, const char *msg);

// The compiled configuration space is split into this many parts per (d_head, dtype); part
// PART of (D, F16) is compiled in its own unit (fa_fwd_inst.hip) and appends its entries.
constexpr int kSpaceParts = 4;
template <int D, bool F16, int PART>
void register_part(AddEntryFn add);

}  // namespace fa
