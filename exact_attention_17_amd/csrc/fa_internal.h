// fa_internal.h -- types shared between the kernel instantiation units and the
// host library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

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
  int n_qtiles;   // ceil(seqlen_q / br)
  int total_wgs;  // batch * heads * n_qtiles
  float scale_log2;  // scale * log2(e): scores go through exp2
};

typedef hipError_t (*LaunchFn)(const FaArgs &, hipStream_t);

// One compiled kernel configuration.
struct KernelEntry {
  int dtype;  // 0 bf16, 1 fp16
  int d_head;
  int br, bc, waves, stages, schedule;
  LaunchFn launch;
  const void *kernel;  // for hipFuncGetAttributes
};

// Each instantiation unit appends its entries.
void register_bf16_d32(void (*add)(const KernelEntry &));
void register_bf16_d64(void (*add)(const KernelEntry &));
void register_bf16_d128(void (*add)(const KernelEntry &));
void register_fp16_d32(void (*add)(const KernelEntry &));
void register_fp16_d64(void (*add)(const KernelEntry &));
void register_fp16_d128(void (*add)(const KernelEntry &));

}  // namespace fa
