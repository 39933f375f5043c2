// fa_bwd.h -- types shared between the backward kernels and the host library (not part of
// the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Backward kernel arguments, passed by value.
struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  const int32_t *cu_seqlens;  // device; nullptr = dense
  int batch, seqlen_q, seqlen_k, heads, heads_kv, group, causal;
  int n_ktiles;   // ceil(seqlen_k / keys per workgroup)
  int total_wgs;  // batch * heads_kv * n_ktiles
  float scale;
  float scale_log2;  // scale * log2(e)
  float *dq_acc;     // [rows, heads, D] fp32, rows = batch * seqlen_q (packed: token rows), for
                     // dQ by atomic adds; nullptr = dQ by the separate pass
  float *dvec;       // [batch, heads, seqlen_q]: D_i = <dO_i, O_i>
  float *lse2;       // [batch, heads, seqlen_q]: L_i log2(e)
};

// Keys per workgroup of the backward kernel for a head dimension.
int bwd_block_keys(int d_head);

// Enqueue the three backward kernels (preprocess, main, dQ conversion).
hipError_t launch_bwd(const BwdArgs &a, int d_head, int dtype, hipStream_t stream);

}  // namespace fa
