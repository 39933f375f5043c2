// fa_fwd_kernel.h -- the gfx950 attention forward kernel (device code).
//
// What it computes: exact attention O = softmax(scale * Q K^T) V and the
// natural-log LSE per query row (page "GPU 内核与 FlashAttention", sections
// 10-11), in the FlashAttention-2 order of that page's section 14: one
// workgroup per (batch, head, query tile of BR rows), an inner loop over
// K/V tiles of BC keys, the running max m, running sum l and unnormalised
// output kept on chip and rescaled by exp(m - m') whenever the max grows
// (section 11.3), O divided by l once at the end and LSE = m + log l stored
// (section 14.1).  Query rows are split among wavefronts, K/V are shared,
// and no wavefront talks to another (section 14.3).  The scale and the max
// subtraction are folded into one FMA feeding exp2 (page "Flash Attention 2
// Chapter6", Kernel 6).
//
// gfx950 mapping (a design of its own; the pages' Ampere fragments,
// ldmatrix and cp.async do not exist here):
//  * Each wavefront owns 32 query rows.  Scores are formed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16 (A = 32 keys x 16 d read from
//    LDS, B = 16 d x 32 queries held in registers for the whole loop).  In
//    the 32x32 accumulator lane l holds query l%32 and 16 of the 32 keys
//    (rows 8g + 4(l/32) + r%4), so a row's max and sum need one exchange
//    between lanes l and l+32 (v_permlane32_swap).
//  * The same registers, rounded to 16 bits, are directly the B operand of
//    O^T = V^T P^T (v_mfma_f32_32x32x16 again).  The key order inside each
//    16-key step is the accumulator's row order; the A operand (V^T, 32 d x
//    16 keys) is read in that order from the row-major V tile with
//    ds_read_b64_tr_b16, which returns four keys of one d column per lane.
//  * K and V tiles go from HBM to LDS with buffer_load_dwordx4 ... lds
//    (no registers, no LDS write instructions); rows past the end of the
//    sequence are out of the buffer's range and read as zero.  Tiles are
//    double buffered: tile j+1 is in flight while tile j is used.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that both the K reads
//    (16 B per lane, 32 rows) and the transposed V reads (8 B per lane,
//    8 rows x 4 chunks) spread over all banks.
//  * Workgroups are renumbered so that the query tiles of one (batch, head)
//    run on the same XCD and share its L2 for K/V.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

// s_waitcnt immediate for "vmcnt(0)" with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int kWaitVmcnt0 = 0x0F70;
// Dword 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const i32x4 &a, const i32x4 &b, const f32x16 &c) {
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 -> two 16-bit values in one dword, round to nearest even.
template <bool F16>
__device__ __forceinline__ int pack2(float x, float y) {
  f32x2 v = {x, y};
  if constexpr (F16) {
    return __builtin_bit_cast(int, __builtin_convertvector(v, f16x2));
  } else {
    return __builtin_bit_cast(int, __builtin_convertvector(v, bf16x2));
  }
}

// XOR mask applied to the 16-byte chunk index of LDS row r (rows of D 16-bit values).
// With C = D/8 chunks per row, it is a bijection of (r / (16/C)) mod C chosen so that
// (a) 16 consecutive rows read at one chunk hit 16 distinct 16-byte bank slots, and
// (b) 4 consecutive rows read at 4 aligned chunks hit 16 distinct slots.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else if constexpr (D == 64) {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  } else {
    return (r >> 2) & 3;
  }
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                           kBufferFlags);
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
fa_fwd_kernel(FaArgs a) {
  constexpr int QW = 32;          // query rows per wavefront
  constexpr int ROWB = D * 2;     // bytes of one row of a tile
  constexpr int TILE = BC * ROWB; // bytes of one K (or V) tile
  constexpr int STAGE = 2 * TILE; // K tile then V tile
  constexpr int NCH = TILE / 1024;  // 1 KB pieces per tile (64 lanes x 16 B)
  constexpr int DT = D / 32;      // 32-wide d tiles of the output
  constexpr int KB = BC / 32;     // 32-key blocks per tile
  constexpr int KS = BC / 16;     // 16-key MFMA steps per tile
  static_assert(BR == NW * QW, "each wavefront owns 32 query rows");
  static_assert(D == 32 || D == 64 || D == 128, "d_head");
  static_assert(BC % 32 == 0 && TILE % 1024 == 0, "tile shape");
  static_assert(STAGES == 1 || STAGES == 2, "stages");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;  // which half of the wavefront

  // Renumber workgroups: hardware deals consecutive ids round-robin over the 8 XCDs,
  // so give XCD x a contiguous range of (batch, head, q-tile) work items.
  const int w = blockIdx.x;
  const int G = a.total_wgs;
  const int per = G >> 3, rem = G & 7, xcd = w & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  const int qt = lin % a.n_qtiles;
  const int bh = lin / a.n_qtiles;
  const int h = bh % a.heads;
  const int b = bh / a.heads;

  int nq, nk;
  int64_t qrow0, krow0;
  if (a.cu_seqlens) {
    const int s0 = a.cu_seqlens[b], s1 = a.cu_seqlens[b + 1];
    nq = nk = s1 - s0;
    qrow0 = krow0 = s0;
  } else {
    nq = a.seqlen_q;
    nk = a.seqlen_k;
    qrow0 = (int64_t)b * nq;
    krow0 = (int64_t)b * nk;
  }
  const int q_tile0 = qt * BR;
  if (q_tile0 >= nq || nk <= 0) return;  // uniform over the workgroup

  const int64_t hd = (int64_t)a.heads * D;
  const uint32_t row_bytes = (uint32_t)(hd * 2);
  const int64_t head_off = (int64_t)h * D;
  const char *qb = (const char *)a.q + (qrow0 * hd + head_off) * 2;
  const char *kb_ = (const char *)a.k + (krow0 * hd + head_off) * 2;
  const char *vb = (const char *)a.v + (krow0 * hd + head_off) * 2;
  char *ob = (char *)a.o + (qrow0 * hd + head_off) * 2;
  const auto rq = make_rsrc(qb, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const auto rk = make_rsrc(kb_, (uint32_t)(nk - 1) * row_bytes + ROWB);
  const auto rv = make_rsrc(vb, (uint32_t)(nk - 1) * row_bytes + ROWB);
  const auto ro = make_rsrc(ob, (uint32_t)(nq - 1) * row_bytes + ROWB);

  // This lane's query row; Q stays in registers as the B operand (16 d per step).
  const int qrow = q_tile0 + wave * QW + (lane & 31);
  i32x4 qreg[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    qreg[t] = __builtin_amdgcn_raw_buffer_load_b128(rq, (uint32_t)qrow * row_bytes + (2 * t + hi) * 16, 0, 0);

  // Issue the loads of K/V tile j into LDS stage st: piece u of a tile is 1 KB, filled by
  // one wavefront instruction; lane i's 16 bytes land at piece + 16 i, so each lane fetches
  // the global chunk that the swizzled layout puts there.
  auto load_tile = [&](int j, int st) {
    char *sk = smem + st * STAGE;
    char *sv = sk + TILE;
    const uint32_t tile_off = (uint32_t)(j * BC) * row_bytes;
#pragma unroll
    for (int i = 0; i < (NCH + NW - 1) / NW; ++i) {
      const int u = wave + i * NW;
      if (NCH % NW == 0 || u < NCH) {
        const int pos = u * 1024 + lane * 16;
        const int r = pos / ROWB;
        const int c = ((pos % ROWB) >> 4) ^ swz<D>(r);
        const uint32_t goff = tile_off + (uint32_t)r * row_bytes + c * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (void FA_LDS *)(sk + u * 1024), 16, goff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (void FA_LDS *)(sv + u * 1024), 16, goff, 0, 0, 0);
      }
    }
  };

  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};
  float m = -INFINITY;  // running max of raw scores (both lanes of a pair hold the same)
  float l = 0.f;        // this lane's share of the running sum of exp2 terms
  const float c = a.scale_log2;

  const int kr = lane & 31;
  const int ksw = swz<D>(kr);
  const int l16 = lane & 15;
  const int g2 = (lane >> 4) & 1;

  const int nkt = (nk + BC - 1) / BC;
  load_tile(0, 0);
  for (int j = 0; j < nkt; ++j) {
    const int st = (STAGES == 2) ? (j & 1) : 0;
    if constexpr (STAGES == 1) {
      if (j > 0) {
        __syncthreads();  // everyone is done with tile j-1
        load_tile(j, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wavefront's pieces of tile j landed
    __syncthreads();                          // ... and everyone's
    if constexpr (STAGES == 2) {
      if (j + 1 < nkt) load_tile(j + 1, (j + 1) & 1);
    }
    const char *sk = smem + st * STAGE;
    const char *sv = sk + TILE;

    // S^T = K_j Q^T for this wavefront's 32 queries: KB accumulators of 32 keys x 32 queries.
    f32x16 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) S[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const i32x4 ka = *(const i32x4 *)(sk + (kb * 32 + kr) * ROWB + (((2 * t + hi) ^ ksw) << 4));
        S[kb] = mfma32<F16>(ka, qreg[t], S[kb]);
      }
    }

    // Keys past the end of the sequence (last tile only) get -inf.
    const int kvalid = nk - j * BC;
    if (kvalid < BC) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) >= kvalid) S[kb][r] = -INFINITY;
    }

    // Online softmax step.
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
        S[kb][r] = p;
        rs += p;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;

    // P~ as 16-bit B operands, one per 16-key step.
    i32x4 P[KS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          P[2 * kb + s2][e] = pack2<F16>(S[kb][8 * s2 + 2 * e], S[kb][8 * s2 + 2 * e + 1]);

    // O^T += V_j^T P~^T.  Lane l's A operand: d = 32 dt + l%32, keys 16 ks + 4(l/32) + {0..3}
    // and 16 ks + 8 + 4(l/32) + {0..3}: two transposed reads, each fed by lanes that point at
    // four rows x 4 consecutive d of the row-major V tile.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = 32 * dt + 16 * g2 + 4 * (l16 & 3);
        const int chunk = col >> 3;
        const int half = l16 & 1;
        const int r0 = 16 * ks + 4 * hi + (l16 >> 2);
        const int r1 = r0 + 8;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 FA_LDS *)(sv + r0 * ROWB + ((chunk ^ swz<D>(r0)) << 4) + half * 8));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 FA_LDS *)(sv + r1 * ROWB + ((chunk ^ swz<D>(r1)) << 4) + half * 8));
        const i16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        O[dt] = mfma32<F16>(__builtin_bit_cast(i32x4, va), P[ks], O[dt]);
      }
    }
  }

  // Epilogue: finish the row sum over the lane pair, normalise, store O and LSE.
  l = pair_sum(l);
  const float inv = 1.f / l;
  if (hi == 0 && qrow < nq) {
    // LSE = scale * m + ln l = ln2 * (m * c + log2 l)
    a.lse[((int64_t)b * a.heads + h) * a.seqlen_q + qrow] =
        0.69314718055994531f * __builtin_fmaf(m, c, __builtin_amdgcn_logf(l));
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // Accumulator groups g0 = 2p, g1 = 2p+1 hold d = 32dt + 8g + 4(l/32) + {0..3}.  After
      // swapping one half-group across the lane pair, lanes < 32 own d = 32dt + 16p + 0..7
      // and lanes >= 32 own d = 32dt + 16p + 8..15.
      const int g0 = 2 * p, g1 = 2 * p + 1;
      const int x0 = pack2<F16>(O[dt][4 * g0 + 0] * inv, O[dt][4 * g0 + 1] * inv);
      const int x1 = pack2<F16>(O[dt][4 * g0 + 2] * inv, O[dt][4 * g0 + 3] * inv);
      const int y0 = pack2<F16>(O[dt][4 * g1 + 0] * inv, O[dt][4 * g1 + 1] * inv);
      const int y1 = pack2<F16>(O[dt][4 * g1 + 2] * inv, O[dt][4 * g1 + 3] * inv);
      auto s0 = __builtin_amdgcn_permlane32_swap((unsigned)x0, (unsigned)y0, false, false);
      auto s1 = __builtin_amdgcn_permlane32_swap((unsigned)x1, (unsigned)y1, false, false);
      const i32x4 out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      const int dcol = 32 * dt + 16 * p + 8 * hi;
      __builtin_amdgcn_raw_buffer_store_b128(out, ro, (uint32_t)qrow * row_bytes + dcol * 2, 0, 0);
    }
  }
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16>
hipError_t launch_fa_fwd(const FaArgs &a, hipStream_t stream) {
  FaArgs arg = a;
  void *args[] = {&arg};
  // hipLaunchKernel reports this launch's own status (hipGetLastError would also return a
  // stale error left by some earlier, unrelated runtime call in this thread).
  return hipLaunchKernel((const void *)&fa_fwd_kernel<D, BR, BC, NW, STAGES, F16>, dim3(a.total_wgs),
                         dim3(NW * 64), args, 0, stream);
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16>
KernelEntry make_entry() {
  KernelEntry e;
  e.dtype = F16 ? 1 : 0;
  e.d_head = D;
  e.br = BR;
  e.bc = BC;
  e.waves = NW;
  e.stages = STAGES;
  e.launch = &launch_fa_fwd<D, BR, BC, NW, STAGES, F16>;
  e.kernel = (const void *)&fa_fwd_kernel<D, BR, BC, NW, STAGES, F16>;
  return e;
}

}  // namespace fa
