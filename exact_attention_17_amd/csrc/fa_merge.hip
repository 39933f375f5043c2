// fa_merge.hip -- combine the partial results of a key range split into num_splits parts.
//
// Split s of a query row holds the attention over its own share of the keys, already
// normalised, O_s, and that share's natural-log LSE_s (-inf, with O_s = 0, when the share had
// no visible key).  The two-block merge of (m, l) of page "GPU 内核与 FlashAttention", section
// 11.2, written for (O, LSE) pairs and any number of parts: with M = max_s LSE_s and
// w_s = exp(LSE_s - M),
//     O = sum_s w_s O_s / sum_s w_s,    LSE = M + ln sum_s w_s.
// At least one split of every row holds key 0, which every row sees, so M is finite.
//
// Memory-bound and small next to the attention itself: each row reads num_splits x (D + 1)
// floats and writes D 16-bit values and one float.  Lane layout: D/4 lanes per row, each
// owning four consecutive d (16-byte loads, 8-byte stores); 256-lane blocks.
#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.h"
#include "fa_internal.h"

namespace fa {

template <int D, bool F16>
__global__ void __launch_bounds__(256) fa_merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;      // lanes per row
  constexpr int RPB = 256 / LPR;  // rows per block
  const int nchunk = (a.seqlen_q + RPB - 1) / RPB;
  const int bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int h = bh % a.heads;
  const int b = bh / a.heads;
  int nq;
  int64_t qrow0;
  if (a.cu_seqlens) {
    qrow0 = a.cu_seqlens[b];
    nq = min(a.cu_seqlens[b + 1] - a.cu_seqlens[b], a.seqlen_q);  // rows past max_seqlen: not used
  } else {
    nq = a.seqlen_q;
    qrow0 = (int64_t)b * nq;
  }
  const int row = chunk * RPB + (int)threadIdx.x / LPR;
  if (row >= nq) return;
  const int c4 = threadIdx.x % LPR;
  const int64_t slab = (int64_t)a.batch * a.heads * a.seqlen_q;  // LSE entries per split
  const int64_t r = ((int64_t)b * a.heads + h) * a.seqlen_q + row;

  // Loads are issued kU splits at a time so that their latencies overlap.  Every split wrote
  // every row below nq (0 and -inf when it had no visible key), so all reads are defined.
  constexpr int kU = 8;
  const int ns = a.num_splits;
  const float *lp = a.lse_part + r;
  const float *op = a.o_part + r * D + 4 * c4;
  float mx = -INFINITY;
  int s = 0;
  for (; s + kU <= ns; s += kU) {
    float t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) t[u] = lp[(s + u) * slab];
#pragma unroll
    for (int u = 0; u < kU; ++u) mx = fmaxf(mx, t[u]);
  }
  for (; s < ns; ++s) mx = fmaxf(mx, lp[s * slab]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float ls, const f32x4 &v) {
    const float wgt = __builtin_amdgcn_exp2f((ls - mx) * 1.4426950408889634f);  // 0 for -inf
    acc += wgt * v;
    wsum += wgt;
  };
  s = 0;
  for (; s + kU <= ns; s += kU) {
    float t[kU];
    f32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      t[u] = lp[(s + u) * slab];
      v[u] = *(const f32x4 *)(op + (s + u) * slab * D);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) add(t[u], v[u]);
  }
  for (; s < ns; ++s) add(lp[s * slab], *(const f32x4 *)(op + s * slab * D));
  const float inv = 1.f / wsum;
  const int lo = pack2<F16>(acc[0] * inv, acc[1] * inv);
  const int hi = pack2<F16>(acc[2] * inv, acc[3] * inv);
  char *orow = (char *)a.o + ((qrow0 + row) * a.heads + h) * (int64_t)(D * 2);
  *(int2 *)(orow + 8 * c4) = make_int2(lo, hi);
  if (c4 == 0) a.lse[r] = mx + 0.69314718055994531f * __builtin_amdgcn_logf(wsum);
}

template <int D, bool F16>
hipError_t launch_merge_t(const MergeArgs &a, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const int nchunk = (a.seqlen_q + RPB - 1) / RPB;
  MergeArgs arg = a;
  void *args[] = {&arg};
  return hipLaunchKernel((const void *)&fa_merge_kernel<D, F16>, dim3(a.batch * a.heads * nchunk), dim3(256),
                         args, 0, stream);
}

hipError_t launch_merge(const MergeArgs &a, int d_head, int dtype, hipStream_t stream) {
  const bool f16 = dtype == 1;
  switch (d_head) {
    case 32:
      return f16 ? launch_merge_t<32, true>(a, stream) : launch_merge_t<32, false>(a, stream);
    case 64:
      return f16 ? launch_merge_t<64, true>(a, stream) : launch_merge_t<64, false>(a, stream);
    case 128:
      return f16 ? launch_merge_t<128, true>(a, stream) : launch_merge_t<128, false>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
