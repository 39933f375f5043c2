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
//  * A block of 32 query rows is the unit of work.  Scores are formed
//    transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = 32 keys x 16 d
//    read from LDS, B = 16 d x 32 queries held in registers for the whole
//    loop).  In the 32x32 accumulator lane l holds query l%32 and 16 of the
//    32 keys (rows 8g + 4(l/32) + r%4), so a row's max and sum need one
//    exchange between lanes l and l+32 (v_permlane32_swap).
//  * The same registers, rounded to 16 bits, are directly the B operand of
//    O^T = V^T P^T (v_mfma_f32_32x32x16 again).  The key order inside each
//    16-key step is the accumulator's row order; the A operand (V^T, 32 d x
//    16 keys) is read in that order from the row-major V tile with
//    ds_read_b64_tr_b16, which returns four keys of one d column per lane.
//  * K and V tiles go from HBM to LDS with buffer_load_dwordx4 ... lds
//    (no registers, no LDS write instructions); rows past the end of the
//    sequence are out of the buffer's range and read as zero.  The next
//    tiles are in flight while the current ones are used.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that both the K reads
//    (16 B per lane, 32 rows) and the transposed V reads (8 B per lane,
//    8 rows x 4 chunks) spread over all banks.
//  * Workgroups are renumbered so that the query tiles of one (batch, K/V
//    head), over all the query heads that share it, run on the same XCD and
//    share its L2 for K/V; an XCD's range runs over K/V heads first, so every
//    XCD gets a share of every (packed) sequence.
//
// Schedules:
//  SCHED 0: each wavefront owns one 32-row block and runs QK^T, softmax and
//    PV of a tile in turn (two wavefronts per SIMD hide each other's stalls).
//    Tiles with no masked key and the others run in separate loops.
//  SCHED 4: SCHED 0 with 32-key tiles at three wavefronts per SIMD (three
//    independent four-wavefront workgroups per CU).  A wavefront's step is a
//    chain of latencies (LDS reads, the matrix results, the row max, the
//    barrier) about twice as long as its own matrix work; a third wavefront
//    per SIMD hides more of it than the shorter tiles cost.
//  SCHED 1: each wavefront owns two 32-row blocks A and B (one wavefront per
//    SIMD, 512 registers) and software-pipelines them so that the softmax of
//    one block (vector ALU) is issued between the matrix instructions of the
//    other: per step j,
//      1. QK_A(j)            alongside  softmax_B(j-1)
//      2. PV_B(j-1)          alongside  softmax_A(j)
//      3. QK_B(j)
//      4. PV_A(j)
//    (the overlap of softmax with matrix work is the point of the ping-pong
//    and intra-warpgroup pipelining of page "GPU 内核与 FlashAttention",
//    sections 15.3-15.4, done here inside one wavefront).  K tiles use a
//    2-slot ring and V tiles a 3-slot ring, since step j reads K(j), V(j) and
//    V(j-1) while K(j+1) and V(j+1) are in flight.
//  SCHED 2: eight wavefronts, each owning one 32-row block, in two groups of
//    four (one wavefront of each group per SIMD).  A workgroup barrier splits
//    every step into a matrix half (PV of the previous tile, QK^T of this
//    one) and a softmax half, and the second group runs one half behind the
//    first: the ping-pong of page "GPU 内核与 FlashAttention", section 15.3,
//    with one barrier in place of named barriers.  The matrix half's two products
//    form one MFMA stream, so LDS reads for QK^T overlap the end of PV.
//  SCHED 5: twelve wavefronts in three groups of four (one of each per SIMD), 32-key
//    tiles, three wavefronts per SIMD.  Barriers split each step into a matrix phase and two
//    softmax phases, and the groups run one phase apart: in every phase one group issues
//    matrix instructions while the other two are in the two parts of their softmax.  A
//    wavefront issues vector instructions at well under the SIMD's rate (about one per 5
//    cycles alone on gfx950; two wavefronts side by side each keep that rate), so giving the
//    softmax two phases and two wavefronts the vector unit keeps it off the critical path.
//    Measured at d_head 128 (16 x 4096 x 16 heads) it is about a tenth slower than SCHED 2:
//    it pays three barriers and a phase hand-off per 32 keys where SCHED 2 pays two per 64,
//    and that costs more than the second vector issuer gains.  The autotuner keeps it in
//    its space.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_internal.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// The running max used as the exponent reference moves only when a tile's row max exceeds
// it by more than this many powers of two (so unnormalised terms stay below 2^8).
constexpr float kLazyRescale = 8.0f;
constexpr float kLazyBound = 256.0f;  // 2^kLazyRescale
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

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Calls f(integral_constant<int, I>) for I = B .. E-1 (indices usable as immediates).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Per-lane LDS read offsets.  With the XOR swizzle they are not affine in the unrolled loop
// indices, but each splits into a per-lane base plus (constant XOR per-lane mask):
//   K operand (t = 16-wide d step, kb = 32-key block):
//     kr*ROWB + (((2t + hi) ^ g) << 4) = kbase + ((32 t) ^ kx) + kb*32*ROWB, g = swz(kr)
//   V^T operand (dt = 32-wide d tile, ks = 16-key step, rho = which four keys):
//     r*ROWB + ((chunk ^ swz(r)) << 4) + 8 half = vbase[rho] + ((64 dt) ^ vx[rho]) + 16 ks*ROWB
// (swz(r) does not depend on ks: the keys of step ks are rows 16 ks + ..., and swz only looks
// at the low four row bits in a way a multiple of 16 leaves alone).
struct LdsAddr {
  int kbase, kx, vbase0, vbase1, vx0, vx1;
};

template <int D>
__device__ __forceinline__ LdsAddr lds_addr(int lane) {
  constexpr int ROWB = D * 2;
  const int kr = lane & 31, hi = (lane >> 5) & 1, l16 = lane & 15, g2 = (lane >> 4) & 1;
  const int gk = swz<D>(kr);
  LdsAddr ad;
  ad.kbase = kr * ROWB + ((hi ^ (gk & 1)) << 4);
  ad.kx = (gk >> 1) << 5;
  const int a = l16 >> 2;                       // row within the four keys of a read
  const int x = 2 * g2 + ((l16 & 3) >> 1);      // chunk within the 32-wide d tile
  const int half = l16 & 1;
  const int r0 = 4 * hi + a, r1 = 8 + 4 * hi + a;
  const int gv0 = swz<D>(r0), gv1 = swz<D>(r1);
  ad.vbase0 = r0 * ROWB + ((x ^ (gv0 & 3)) << 4) + half * 8;
  ad.vbase1 = r1 * ROWB + ((x ^ (gv1 & 3)) << 4) + half * 8;
  ad.vx0 = (gv0 >> 2) << 6;
  ad.vx1 = (gv1 >> 2) << 6;
  return ad;
}

// LDS reads as inline assembly.  The compiler neither knows which LDS bytes a transposing
// read touches (it would otherwise wait for every LDS DMA in flight, the prefetch of later
// tiles, before each one) nor keeps enough reads in flight ahead of the MFMAs that consume
// them; so reads are issued here a fixed distance ahead and their completion is awaited
// explicitly.  LDS operations complete in issue order, so "at most N outstanding" means all
// but the N most recent reads are done.  lds_dep makes a register look redefined after the
// wait, so that its consumer cannot be scheduled above the wait.
template <int OFF>
__device__ __forceinline__ void lds_read_b128(i32x4 &r, uint32_t addr) {
  __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read_tr(i16x4 &r, uint32_t addr) {
  __asm__ volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  __asm__ volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}
template <typename T>
__device__ __forceinline__ void lds_dep(T &r) {
  __asm__ volatile("" : "+v"(r));
}

template <int V>
using IC = std::integral_constant<int, V>;

// S^T = K_tile Q^T for one 32-query block: KB accumulators of 32 keys x 32 queries.  MFMA i
// (t = i / KB, kb = i % KB) reads its K operand LA reads ahead.
// SOFF is a byte offset from sk carried in the reads' immediate field, so that the per-lane
// addresses (one register per d step) do not depend on which ring slot is read.
template <int D, int BC, bool F16, int LA = 6, int SOFF = 0>
__device__ __forceinline__ void qk_block(const char *sk, f32x16 (&S)[BC / 32], const i32x4 (&qr)[D / 16],
                                         const LdsAddr &ad) {
  constexpr int ROWB = D * 2, KB = BC / 32, T = D / 16, N = T * KB;
  static_assert(SOFF + (KB - 1) * 32 * ROWB < 65536, "ds_read offset field");
  constexpr int L = LA < N ? LA : N;
  const uint32_t sk_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sk;
  uint32_t koff[T];
#pragma unroll
  for (int t = 0; t < T; ++t) koff[t] = sk_lds + (uint32_t)(((32 * t) ^ ad.kx) + ad.kbase);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) S[kb] = f32x16{};
  i32x4 buf[L + 1];
  auto issue = [&buf, &koff](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    lds_read_b128<SOFF + (i % KB) * 32 * ROWB>(buf[i % (L + 1)], koff[i / KB]);
  };
  static_for<0, L>(issue);
  static_for<0, N>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if constexpr (i + L < N) issue(IC<i + L>{});
    constexpr int after = (N - 1 - i) < L ? (N - 1 - i) : L;  // reads issued after read i
    lds_wait<after>();
    lds_dep(buf[i % (L + 1)]);
    S[i % KB] = mfma32<F16>(buf[i % (L + 1)], qr[i / KB], S[i % KB]);
  });
}

// O^T += V_tile^T P~^T for one 32-query block.  Lane l's A operand: d = 32 dt + l%32, keys
// 16 ks + 4(l/32) + {0..3} and 16 ks + 8 + 4(l/32) + {0..3}: two transposed reads, each fed
// by lanes that point at four rows x 4 consecutive d of the row-major V tile.  MFMA i
// (ks = i / DT, dt = i % DT) has its two reads issued LA MFMAs ahead.
// (SOFF as in qk_block)
template <int D, int BC, bool F16, int LA = 4, int SOFF = 0>
__device__ __forceinline__ void pv_block(const char *sv, const i32x4 (&P)[BC / 16], f32x16 (&O)[D / 32],
                                         const LdsAddr &ad) {
  constexpr int ROWB = D * 2, DT = D / 32, KS = BC / 16, N = KS * DT;
  constexpr int L = LA < N ? LA : N;
  static_assert(SOFF + 16 * (KS - 1) * ROWB < 65536, "ds_read offset field");
  static_assert(2 * L <= 15, "lgkmcnt field");
  const uint32_t sv_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sv;
  uint32_t a0[DT], a1[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    a0[dt] = sv_lds + (uint32_t)(((64 * dt) ^ ad.vx0) + ad.vbase0);
    a1[dt] = sv_lds + (uint32_t)(((64 * dt) ^ ad.vx1) + ad.vbase1);
  }
  i16x4 b0[L + 1], b1[L + 1];
  auto issue = [&b0, &b1, &a0, &a1](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    lds_read_tr<SOFF + 16 * (i / DT) * ROWB>(b0[i % (L + 1)], a0[i % DT]);
    lds_read_tr<SOFF + 16 * (i / DT) * ROWB>(b1[i % (L + 1)], a1[i % DT]);
  };
  static_for<0, L>(issue);
  static_for<0, N>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if constexpr (i + L < N) issue(IC<i + L>{});
    constexpr int after = 2 * ((N - 1 - i) < L ? (N - 1 - i) : L);  // reads issued after MFMA i's
    lds_wait<after>();
    lds_dep(b0[i % (L + 1)]);
    lds_dep(b1[i % (L + 1)]);
    const i16x4 &v0 = b0[i % (L + 1)], &v1 = b1[i % (L + 1)];
    const i16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    O[i % DT] = mfma32<F16>(__builtin_bit_cast(i32x4, va), P[i / DT], O[i % DT]);
  });
}

// Reads still outstanding after those of op I in a stream of N ops whose op k has its reads
// issued before op k - L: ops I+1 .. min(I+L, N-1), two reads for a PV op (k < NP), one for a
// QK^T op.
template <int I, int L, int N, int NP>
constexpr int pvqk_after() {
  int n = 0;
  for (int k = I + 1; k <= I + L && k < N; ++k) n += k < NP ? 2 : 1;
  return n;
}

// PV of the previous tile (pv_block) and S^T = K Q^T of this one (qk_block) as one stream of
// MFMAs with one read lookahead, so that the first K reads are in flight during the last PV
// MFMAs rather than issued after them.  Same products in the same order as the two
// functions called in turn.
template <int D, int BC, bool F16, int LA, int SOFFV, int SOFFK>
__device__ __forceinline__ void pvqk_block(const char *sv, const i32x4 (&P)[BC / 16], f32x16 (&O)[D / 32],
                                           const char *sk, f32x16 (&S)[BC / 32], const i32x4 (&qr)[D / 16],
                                           const LdsAddr &ad) {
  constexpr int ROWB = D * 2, DT = D / 32, KS = BC / 16, NP = KS * DT, KB = BC / 32, T = D / 16;
  constexpr int N = NP + T * KB, L = LA < N ? LA : N;
  static_assert(2 * L <= 15, "lgkmcnt field");
  static_assert(SOFFV + 16 * (KS - 1) * ROWB < 65536 && SOFFK + (KB - 1) * 32 * ROWB < 65536,
                "ds_read offset field");
  const uint32_t sv_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sv;
  const uint32_t sk_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sk;
  uint32_t a0[DT], a1[DT], koff[T];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    a0[dt] = sv_lds + (uint32_t)(((64 * dt) ^ ad.vx0) + ad.vbase0);
    a1[dt] = sv_lds + (uint32_t)(((64 * dt) ^ ad.vx1) + ad.vbase1);
  }
#pragma unroll
  for (int t = 0; t < T; ++t) koff[t] = sk_lds + (uint32_t)(((32 * t) ^ ad.kx) + ad.kbase);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) S[kb] = f32x16{};
  i16x4 b0[L + 1], b1[L + 1];
  i32x4 kbuf[L + 1];
  auto issue = [&](auto k_c) __attribute__((always_inline)) {
    constexpr int k = decltype(k_c)::value;
    if constexpr (k < NP) {
      lds_read_tr<SOFFV + 16 * (k / DT) * ROWB>(b0[k % (L + 1)], a0[k % DT]);
      lds_read_tr<SOFFV + 16 * (k / DT) * ROWB>(b1[k % (L + 1)], a1[k % DT]);
    } else {
      constexpr int i = k - NP;
      lds_read_b128<SOFFK + (i % KB) * 32 * ROWB>(kbuf[k % (L + 1)], koff[i / KB]);
    }
  };
  static_for<0, L>(issue);
  static_for<0, N>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if constexpr (i + L < N) issue(IC<i + L>{});
    lds_wait<pvqk_after<i, L, N, NP>()>();
    if constexpr (i < NP) {
      lds_dep(b0[i % (L + 1)]);
      lds_dep(b1[i % (L + 1)]);
      const i16x4 &v0 = b0[i % (L + 1)], &v1 = b1[i % (L + 1)];
      const i16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      O[i % DT] = mfma32<F16>(__builtin_bit_cast(i32x4, va), P[i / DT], O[i % DT]);
    } else {
      constexpr int q = i - NP;
      lds_dep(kbuf[i % (L + 1)]);
      S[q % KB] = mfma32<F16>(kbuf[i % (L + 1)], qr[q / KB], S[q % KB]);
    }
  });
}

// A lane's share of a row sum over one tile, term i being accumulator register i % 16 of
// 32-key block i / 16.  It is accumulated in four interleaved partial sums (term i goes to
// sum i % 4), added pairwise at the end: four short chains of dependent adds instead of one
// long one (about 0.5 % on the ping-pong schedule; on 32-key tiles 0.6 % under the causal
// mask and 0.8-1.4 % at d_head 32).
struct RowSum {
  static constexpr int NP = 4;
  float v[NP];
  // the first NP terms start the sums (0 + x is x exactly for these terms, all >= 0)
  __device__ __forceinline__ void add(int i, float x) {
    if (i < NP)
      v[i] = x;
    else
      v[i % NP] += x;
  }
  __device__ __forceinline__ float total() const { return (v[0] + v[1]) + (v[2] + v[3]); }
};

// Online softmax step of one 32-query block on the raw scores S of tile j (keys from
// kvalid on, when MASK, are past the sequence end).  Leaves P~ (16-bit PV operands) in P,
// updates m and l, and returns alpha, the factor O must be multiplied by before this tile's
// PV; rescale is false when no row of the wavefront needs it (alpha is then 1 everywhere).
// The reference max m only moves when this tile's row max exceeds it by more than
// kLazyRescale in exp2 units; otherwise the exponentials are taken against the old m (they
// stay below 2^kLazyRescale), and the rescale of O and l, an exact identity whichever
// reference is used, is skipped.
template <int BC, bool F16, bool MASK>
__device__ __forceinline__ float softmax_block(f32x16 (&S)[BC / 32], i32x4 (&P)[BC / 16], float &m, float &l,
                                               float c, int kvalid_lane, bool &rescale) {
  constexpr int KB = BC / 32;
  if constexpr (MASK) {
    // key of accumulator register r in block kb is kb*32 + 8(r/4) + 4 hi + r%4; the lane part
    // 4 hi is already taken off kvalid_lane so that the compared constants are immediates
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) >= kvalid_lane) S[kb][r] = -INFINITY;
  }
  float mx = S[0][0];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
  mx = pair_max(mx);
  const bool grow = (mx - m) * c > kLazyRescale;  // true at the first visible key (m = -inf)
  const float m_new = grow ? mx : m;
  // m_new stays -inf while a row has seen no visible key (a split of the key range that lies
  // wholly above the diagonal for it); the exponentials are then taken against 0 and are 0.
  const float m_ref = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f((m - m_ref) * c);  // 0 on the first tile, else <= 1
  rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
  m = m_new;
  const float mc = m_ref * c;
  RowSum rs;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
      S[kb][r] = p;
      rs.add(16 * kb + r, p);
    }
  l = l * alpha + rs.total();
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        P[2 * kb + s2][e] = pack2<F16>(S[kb][8 * s2 + 2 * e], S[kb][8 * s2 + 2 * e + 1]);
  return alpha;
}

// The same step for a tile with no masked key, speculating that the reference max stays:
// the exponentials are first taken against the current m.  If every lane's partial sum of
// them is at most 2^kLazyRescale, so is each of them (all are >= 0), so no row's max moved
// by more than kLazyRescale and the step above would have kept m: the result is then bit
// for bit the same (same products, same order of sums, alpha = 1).  Otherwise (in
// particular on a row's first tile, where m = -inf makes the sum +inf or NaN) the step
// above is taken from the scores, into the same registers.  The row max and its exchange
// between lanes leave the common path.
template <int BC, bool F16>
__device__ __forceinline__ float softmax_block_spec(const f32x16 (&S)[BC / 32], i32x4 (&P)[BC / 16], float &m,
                                                    float &l, float c, bool &rescale) {
  constexpr int KB = BC / 32;
  f32x16 E[KB];
  float mc = m * c;
  RowSum part;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      E[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
      part.add(16 * kb + r, E[kb][r]);
    }
  float rs = part.total();
  float alpha = 1.f;
  rescale = false;
  if (__builtin_amdgcn_ballot_w64(!(rs <= kLazyBound)) != 0) {
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = pair_max(mx);
    const bool grow = (mx - m) * c > kLazyRescale;
    const float m_new = grow ? mx : m;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    alpha = __builtin_amdgcn_exp2f((m - m_ref) * c);
    rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
    m = m_new;
    mc = m_ref * c;
    RowSum again;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        E[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
        again.add(16 * kb + r, E[kb][r]);
      }
    rs = again.total();
  }
  l = l * alpha + rs;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        P[2 * kb + s2][e] = pack2<F16>(E[kb][8 * s2 + 2 * e], E[kb][8 * s2 + 2 * e + 1]);
  return alpha;
}

// The speculative step without a second copy of the scores, for schedules whose registers
// cannot hold one: the exponentials overwrite S.  When the partial-sum test fails (always on
// a row's first tile, where m = -inf makes the sum +inf), `rescore` forms the scores again
// from the K tile still in LDS and the step continues as the plain one.  The result is the
// plain step's, bit for bit, as for softmax_block_spec.
template <int BC, bool F16, typename Rescore>
__device__ __forceinline__ float softmax_block_spec_inplace(f32x16 (&S)[BC / 32], i32x4 (&P)[BC / 16], float &m,
                                                            float &l, float c, bool &rescale, Rescore &&rescore) {
  constexpr int KB = BC / 32;
  float mc = m * c;
  RowSum part;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
      part.add(16 * kb + r, S[kb][r]);
    }
  float rs = part.total();
  float alpha = 1.f;
  rescale = false;
  if (__builtin_amdgcn_ballot_w64(!(rs <= kLazyBound)) != 0) {
    rescore(S);
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = pair_max(mx);
    const bool grow = (mx - m) * c > kLazyRescale;
    const float m_new = grow ? mx : m;
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    alpha = __builtin_amdgcn_exp2f((m - m_ref) * c);
    rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
    m = m_new;
    mc = m_ref * c;
    RowSum again;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -mc));
        again.add(16 * kb + r, S[kb][r]);
      }
    rs = again.total();
  }
  l = l * alpha + rs;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        P[2 * kb + s2][e] = pack2<F16>(S[kb][8 * s2 + 2 * e], S[kb][8 * s2 + 2 * e + 1]);
  return alpha;
}

template <int DT>
__device__ __forceinline__ void rescale_o(f32x16 (&O)[DT], float alpha) {
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
}

// Finish one 32-query block: total the row sum over the lane pair, normalise, store O (16-bit)
// and LSE.  qrow0 is the block's first row in the sequence.
template <int D, bool F16>
__device__ __forceinline__ void store_block(const f32x16 (&O)[D / 32], float m, float l, float c, int qrow0,
                                            int nq, uint32_t row_bytes, const __amdgpu_buffer_rsrc_t &ro,
                                            float *lse_row, int lane) {
  constexpr int DT = D / 32;
  const int hi = lane >> 5;
  l = pair_sum(l);
  const float inv = 1.f / l;
  const int qrow = qrow0 + (lane & 31);
  if (hi == 0 && qrow < nq) {
    // LSE = scale * m + ln l = ln2 * (m * c + log2 l)
    lse_row[qrow] = 0.69314718055994531f * __builtin_fmaf(m, c, __builtin_amdgcn_logf(l));
  }
  const uint32_t o_off = (uint32_t)qrow * row_bytes + hi * 16;
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
      // rows past nq are out of the buffer's range: the store is dropped
      __builtin_amdgcn_raw_buffer_store_b128(out, ro, o_off + (32 * dt + 16 * p) * 2, 0, 0);
    }
  }
}

// Split-mode finish of one 32-query block: the split's own normalised output in fp32 and its
// natural-log LSE, or 0 and -inf for a row that saw no visible key.  rp covers this (split,
// batch, head)'s [rows < nq, D] fp32 slab; lane l holds d = 32 dt + 8 g + 4 (l/32) + 0..3 of
// row l % 32, four consecutive floats, stored as they are.
template <int D>
__device__ __forceinline__ void store_block_part(const f32x16 (&O)[D / 32], float m, float l, float c,
                                                 int qrow0, int nq, const __amdgpu_buffer_rsrc_t &rp,
                                                 float *lse_row, int lane) {
  constexpr int DT = D / 32;
  const int hi = lane >> 5;
  l = pair_sum(l);
  const bool seen = l > 0.f;
  const float inv = seen ? 1.f / l : 0.f;
  const int qrow = qrow0 + (lane & 31);
  if (hi == 0 && qrow < nq)
    lse_row[qrow] = seen ? 0.69314718055994531f * __builtin_fmaf(m, c, __builtin_amdgcn_logf(l)) : -INFINITY;
  const uint32_t off = (uint32_t)qrow * (D * 4) + hi * 16;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 val = {O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv, O[dt][4 * g + 2] * inv,
                         O[dt][4 * g + 3] * inv};
      // rows past nq are out of the buffer's range: the store is dropped
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, val), rp, off + (32 * dt + 8 * g) * 4, 0, 0);
    }
}

template <int SCHED>
constexpr int waves_per_simd() {
  return SCHED == 1 ? 1 : (SCHED == 4 || SCHED == 5) ? 3 : 2;
}

// Workgroup barrier without the memory fences of __syncthreads (which would also wait for
// the LDS DMA of later tiles still in flight); the empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16, int SCHED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<SCHED>())))
fa_fwd_kernel(FaArgs a) {
  constexpr int NB = SCHED == 1 ? 2 : 1;  // 32-query blocks per wavefront
  constexpr int QW = 32 * NB;             // query rows per wavefront
  constexpr int ROWB = D * 2;             // bytes of one row of a tile
  constexpr int TILE = BC * ROWB;         // bytes of one K (or V) tile
  constexpr int NCH = TILE / 1024;        // 1 KB pieces per tile (64 lanes x 16 B)
  constexpr int DT = D / 32;              // 32-wide d tiles of the output
  constexpr int KB = BC / 32;             // 32-key blocks per tile
  constexpr int KS = BC / 16;             // 16-key MFMA steps per tile
  // LDS: SCHED 0 holds STAGES (K, V) tile pairs; SCHED 1 a 2-slot K ring and a 3-slot V ring;
  // SCHED 2 (STAGES = 3) a 3-slot V ring and a 3-slot K ring.
  constexpr int LDS_BYTES = SCHED == 1 ? 5 * TILE : STAGES * 2 * TILE;
  static_assert(BR == NW * QW, "rows per workgroup");
  static_assert(D == 32 || D == 64 || D == 128, "d_head");
  static_assert(BC % 32 == 0 && TILE % 1024 == 0, "tile shape");
  static_assert(STAGES >= 1 && STAGES <= 4, "stages");
  static_assert(SCHED == 0 || (SCHED == 1 && STAGES == 2) || (SCHED == 2 && STAGES == 3 && NW == 8) ||
                    (SCHED == 4 && BC == 32) || (SCHED == 5 && STAGES == 3 && NW == 12),
                "schedule");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;  // which half of the wavefront

  // Renumber workgroups: hardware deals consecutive ids round-robin over the 8 XCDs,
  // so give XCD x a contiguous range of (batch, head, q-tile, split) work items.
  const int w = blockIdx.x;
  const int G = a.total_wgs;
  const int per = G >> 3, rem = G & 7, xcd = w & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  // (divisions by the launch's fixed divisors: multiply-high, add, shift)
  const int nsplit = a.num_splits;
  const int lt = (int)fast_div((uint32_t)lin, a.div_splits);
  const int split = lin - lt * nsplit;
  const int ght = (int)fast_div((uint32_t)lt, a.div_qtiles);
  const int qi = lt - ght * a.n_qtiles;
  // under the causal mask the work of a query tile grows with its index: start the longest
  const int qt = a.causal ? a.n_qtiles - 1 - qi : qi;
  // head-major: an XCD's contiguous range covers a few K/V heads of every sequence, so packed
  // sequences of different lengths spread evenly over the XCDs, while the query tiles of one
  // (sequence, K/V head) -- of all the query heads that share it -- stay together and share
  // that XCD's L2 for their K/V.  Order: (K/V head, sequence, head in group, query tile).
  const int hkb = (int)fast_div((uint32_t)ght, a.div_group);
  const int gi = ght - hkb * a.group;
  // Dense calls whose head rows are under 128 bytes (d_head 32) take the sequence outermost
  // instead, so that the heads sharing a cache line of a token row are read by workgroups
  // running at the same time (2.5 % on B64 N512 H16 d32, which fetches about twice its
  // input bytes from HBM).
  const bool seq_major = D * 2 < 128 && !a.cu_seqlens;
  const int hkq = (int)fast_div((uint32_t)hkb, seq_major ? a.div_heads_kv : a.div_batch);
  const int b = seq_major ? hkq : hkb - hkq * a.batch;
  const int hk = seq_major ? hkb - hkq * a.heads_kv : hkq;  // the K/V head this query head reads
  const int h = hk * a.group + gi;

  int nq, nk;
  int64_t qrow0, krow0;
  if (a.cu_seqlens) {
    // a sequence longer than max_seqlen (the LSE row pitch) breaks the caller's contract;
    // only its first max_seqlen tokens are used, so no access leaves the buffers
    const int s0 = a.cu_seqlens[b], s1 = a.cu_seqlens[b + 1];
    nq = nk = min(s1 - s0, a.seqlen_q);
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
  const int64_t hkd = (int64_t)a.heads_kv * D;
  const uint32_t row_bytes = (uint32_t)(hd * 2);
  const uint32_t kv_row_bytes = (uint32_t)(hkd * 2);
  const char *qb = (const char *)a.q + (qrow0 * hd + (int64_t)h * D) * 2;
  const char *kb_ = (const char *)a.k + (krow0 * hkd + (int64_t)hk * D) * 2;
  const char *vb = (const char *)a.v + (krow0 * hkd + (int64_t)hk * D) * 2;
  char *ob = (char *)a.o + (qrow0 * hd + (int64_t)h * D) * 2;
  const auto rq = make_rsrc(qb, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const auto ro = make_rsrc(ob, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const int64_t lse_base = ((int64_t)b * a.heads + h) * a.seqlen_q;
  float *lse_row = a.lse + lse_base;
  // split mode: this split's fp32 slab [rows < nq, D] and its LSE row
  const int64_t part_base = (int64_t)split * a.batch * a.heads * a.seqlen_q + lse_base;
  float *lse_part_row = a.lse_part + part_base;
  const auto rp = make_rsrc(a.o_part + part_base * D, (uint32_t)nq * (D * 4));

  // Key tiles this workgroup visits: [0, nk), or under the causal mask those up to the
  // tile's last query row (the rest lie wholly above the diagonal and are skipped); split
  // `split` of nsplit takes tiles [jb, je) of them.
  const int kend = a.causal ? min(nk, q_tile0 + BR) : nk;
  const int nkt_all = (kend + BC - 1) / BC;
  const int jb = nsplit == 1 ? 0 : (int)((int64_t)nkt_all * split / nsplit);
  const int je = nsplit == 1 ? nkt_all : (int)((int64_t)nkt_all * (split + 1) / nsplit);
  const int ntl = je - jb;  // may be 0: the split then reports "no visible key"

  // Q stays in registers as the B operand (16 d per step) of each 32-row block.
  const int wrow0 = q_tile0 + wave * QW;  // first row of this wavefront
  i32x4 qreg[NB][D / 16];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      qreg[nb][t] = __builtin_amdgcn_raw_buffer_load_b128(
          rq, (uint32_t)(wrow0 + 32 * nb + (lane & 31)) * row_bytes + (2 * t + hi) * 16, 0, 0);

  // Issue the loads of tile j of K (or V) into LDS at dst: piece u of a tile is 1 KB, filled
  // by one wavefront instruction; lane i's 16 bytes land at piece + 16 i, so each lane
  // fetches the global chunk that the swizzled layout puts there.  LW wavefronts share the
  // pieces, this one being number lw among them.
  // The tile's offset goes into the buffer resource (base advanced, range shortened: scalar
  // work) rather than into every lane's offset, so that the per-lane offsets are the same for
  // every tile and no vector instruction is spent on them.  The range check still bounds the
  // sequence: tile j starts below its end (it holds a key), and rows past the end read as zero.
  const uint32_t kv_bytes = (uint32_t)(nk - 1) * kv_row_bytes + ROWB;
  auto load_by = [&](const char *base, char *dst, int j, int lw, auto lw_c) __attribute__((always_inline)) {
    constexpr int LW = decltype(lw_c)::value;
    const uint32_t tile_off = (uint32_t)(j * BC) * kv_row_bytes;
    const auto rsrc = make_rsrc(base + tile_off, kv_bytes - tile_off);
#pragma unroll
    for (int i = 0; i < (NCH + LW - 1) / LW; ++i) {
      const int u = lw + i * LW;
      if (NCH % LW == 0 || u < NCH) {
        const int pos = u * 1024 + lane * 16;
        const int r = pos / ROWB;
        const int cc = ((pos % ROWB) >> 4) ^ swz<D>(r);
        const uint32_t goff = (uint32_t)r * kv_row_bytes + cc * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void FA_LDS *)(dst + u * 1024), 16, goff, 0, 0, 0);
      }
    }
  };
  auto load_one = [&](const char *base, char *dst, int j) __attribute__((always_inline)) {
    load_by(base, dst, j, wave, std::integral_constant<int, NW>{});
  };

  f32x16 O[NB][DT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[nb][dt] = f32x16{};
  float m[NB], l[NB];  // running max of raw scores (same on both lanes of a pair); lane's sum share
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.f;
  }
  const float c = a.scale_log2;
  const LdsAddr ad = lds_addr<D>(lane);

  // Masking per 32-row block nb: tiles below kfull[nb] hold no masked key for any row of the
  // block; in the others, lane's row sees keys below klim[nb] (the sequence end, and under
  // the causal mask its own index + 1).  Keys from wave_kend on are masked for every row of
  // the wavefront.
  int kfull[NB], klim[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r0 = wrow0 + 32 * nb;
    kfull[nb] = (a.causal ? min(nk, r0 + 1) : nk) / BC;
    klim[nb] = a.causal ? min(nk, r0 + (lane & 31) + 1) : nk;
  }
  const int wave_kend = a.causal ? min(nk, wrow0 + QW) : nk;
  auto softmax = [&](f32x16 (&S)[KB], i32x4 (&P)[KS], int nb, int j, bool &rescale) __attribute__((always_inline)) {
    if (j < kfull[nb]) return softmax_block<BC, F16, false>(S, P, m[nb], l[nb], c, 0, rescale);
    return softmax_block<BC, F16, true>(S, P, m[nb], l[nb], c, klim[nb] - j * BC - 4 * hi, rescale);
  };
  auto finish = [&](int nb) __attribute__((always_inline)) {
    if (nsplit > 1)
      store_block_part<D>(O[nb], m[nb], l[nb], c, wrow0 + 32 * nb, nq, rp, lse_part_row, lane);
    else
      store_block<D, F16>(O[nb], m[nb], l[nb], c, wrow0 + 32 * nb, nq, row_bytes, ro, lse_row, lane);
  };

  if constexpr (SCHED == 0 || SCHED == 4) {
    // (schedule 4 is this loop at three wavefronts per SIMD: 32-key tiles and shorter LDS
    // read lookahead keep a lane within 168 registers)
    constexpr int QK_LA = SCHED == 4 ? 3 : 6, PV_LA = SCHED == 4 ? 2 : 4;
    // STAGES (K, V) tile pairs in LDS, tile j in stage j % STAGES; tile j + STAGES - 1 is
    // requested at the start of step j (its stage held tile j - 1, which every wavefront
    // finished before the barrier that opens step j), so STAGES - 1 tiles are in flight.
    constexpr int STAGE = 2 * TILE;  // K tile then V tile
    constexpr int LPT = 2 * (NCH >= NW ? NCH / NW : 1);  // loads per tile of a loading wavefront
    static_assert(NCH % NW == 0 || NW % NCH == 0, "tile pieces spread evenly");
    // MODE 0: no masked key in the tile, speculative softmax; 1: the tile may hold masked
    // keys; 2: no masked key, and the tile is the workgroup's first (m is still -inf, so the
    // speculation would fail and the exponentials be taken twice; O is still zero, so its
    // rescale by alpha = 0 is left out).
    auto step = [&](auto st_c, auto mode_c, int j) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr int MODE = decltype(mode_c)::value;
      constexpr bool MK = MODE == 1;
      if constexpr (STAGES == 1) {
        if (j > 0) {
          __syncthreads();  // everyone is done with tile j-1
          load_one(kb_, smem, jb + j);
          load_one(vb, smem + TILE, jb + j);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      } else {
        // this wavefront's pieces of tile j landed: at most the later tiles' loads pending
        const int ahead = min(STAGES - 2, ntl - 1 - j);
        if (ahead <= 0) {
          wait_vmcnt<0>();
        } else if constexpr (STAGES < 4) {
          wait_vmcnt<LPT>();
        } else {
          if (ahead == 1)
            wait_vmcnt<LPT>();
          else
            wait_vmcnt<2 * LPT>();
        }
      }
      wg_barrier();  // ... and everyone's; and everyone is done with tile j - 1
      if constexpr (STAGES >= 2) {
        constexpr int NS = (ST + STAGES - 1) % STAGES;  // stage of tile j + STAGES - 1
        if (j + STAGES - 1 < ntl) {
          load_one(kb_, smem + NS * STAGE, jb + j + STAGES - 1);
          load_one(vb, smem + NS * STAGE + TILE, jb + j + STAGES - 1);
        }
      }
      // (an unmasked tile has a key visible to every row of the wavefront; a masked one may
      // have none, and is then skipped)
      if (!MK || (jb + j) * BC < wave_kend) {
        f32x16 S[KB];
        i32x4 P[KS];
        bool rs;
        // the slot's offset goes into the reads' immediate field when it fits
        constexpr int SO = ST * STAGE;
        constexpr bool IMM = SO + STAGE <= 65536;
        const char *base = IMM ? smem : smem + SO;
        qk_block<D, BC, F16, QK_LA, IMM ? SO : 0>(base, S, qreg[0], ad);
        // (schedule 4 speculates in place: a second copy of the scores spills there)
        auto rescore = [&](f32x16(&S2)[KB]) __attribute__((always_inline)) {
          qk_block<D, BC, F16, QK_LA, IMM ? SO : 0>(base, S2, qreg[0], ad);
        };
        const float alpha =
            MODE != 0 ? softmax_block<BC, F16, MK>(S, P, m[0], l[0], c, MK ? klim[0] - (jb + j) * BC - 4 * hi : 0, rs)
            : SCHED == 4 ? softmax_block_spec_inplace<BC, F16>(S, P, m[0], l[0], c, rs, rescore)
                         : softmax_block_spec<BC, F16>(S, P, m[0], l[0], c, rs);
        if (MODE != 2 && rs) rescale_o<DT>(O[0], alpha);
        pv_block<D, BC, F16, PV_LA, (IMM ? SO : 0) + TILE>(base, P, O[0], ad);
      }
    };
    // Tiles [0, jm) hold no masked key for this wavefront, tiles [jm, ntl) may.  Each range
    // runs in a loop of its own: with one loop and a branch around the masking, the scores
    // (or, with the branch around the whole tile, the output accumulators) of the two paths
    // meet at the end of every step and the compiler copies all of them between registers.
    const int jm = min(max(kfull[0] - jb, 0), ntl);
    auto run = [&](auto mode_c, int j0, int j1) __attribute__((always_inline)) {
      for (int jj = j0 - j0 % STAGES; jj < j1; jj += STAGES) {
        static_for<0, STAGES>([&](auto st_c) __attribute__((always_inline)) {
          const int j = jj + decltype(st_c)::value;
          if (j >= j0 && j < j1) step(st_c, mode_c, j);
        });
      }
    };
#pragma unroll
    for (int t = 0; t < (STAGES > 1 ? STAGES - 1 : 1); ++t) {
      if (t < ntl) {
        load_one(kb_, smem + t * STAGE, jb + t);
        load_one(vb, smem + t * STAGE + TILE, jb + t);
      }
    }
    if (jm > 0) {
      step(IC<0>{}, IC<2>{}, 0);
      run(IC<0>{}, 1, jm);
    }
    run(IC<1>{}, jm, ntl);
    finish(0);
  } else if constexpr (SCHED == 1) {
    // Dual-block software pipeline (see the header comment).  Step j:
    //   issue loads K(j+1) -> K slot (j+1)%2 (held K(j-1), last read in step j-1) and
    //                V(j+1) -> V slot (j+1)%3 (held V(j-2), last read in step j-1);
    //   1. QK_A(j) [K slot j%2]            with softmax_B(j-1)
    //   2. PV_B(j-1) [V slot (j-1)%3]      with softmax_A(j)
    //   3. QK_B(j) [K slot j%2]
    //   4. PV_A(j) [V slot j%3]
    // Loads issued at the start of step j are waited for at the start of step j+1.
    f32x16 S[2][KB];
    i32x4 P[2][KS];
    float alpha[2] = {1.f, 1.f};
    bool rs[2] = {false, false};
    auto kslot = [&](int j) __attribute__((always_inline)) { return smem + (j & 1) * TILE; };
    auto vslot = [&](int j) __attribute__((always_inline)) { return smem + 2 * TILE + (j % 3) * TILE; };
    if (ntl > 0) {
      load_one(kb_, kslot(0), jb);
      load_one(vb, vslot(0), jb);
    }
    for (int j = 0; j <= ntl; ++j) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (j + 1 < ntl) {
        load_one(kb_, kslot(j + 1), jb + j + 1);
        load_one(vb, vslot(j + 1), jb + j + 1);
      }
      // 1.
      if (j < ntl) qk_block<D, BC, F16>(kslot(j), S[0], qreg[0], ad);
      if (j >= 1) alpha[1] = softmax(S[1], P[1], 1, jb + j - 1, rs[1]);
      __builtin_amdgcn_sched_barrier(0);
      // 2.
      if (j >= 1) {
        if (rs[1]) rescale_o<DT>(O[1], alpha[1]);
        pv_block<D, BC, F16>(vslot(j - 1), P[1], O[1], ad);
      }
      if (j < ntl) alpha[0] = softmax(S[0], P[0], 0, jb + j, rs[0]);
      __builtin_amdgcn_sched_barrier(0);
      // 3. and 4.
      if (j < ntl) {
        qk_block<D, BC, F16>(kslot(j), S[1], qreg[1], ad);
        if (rs[0]) rescale_o<DT>(O[0], alpha[0]);
        pv_block<D, BC, F16>(vslot(j), P[0], O[0], ad);
      }
    }
    finish(0);
    finish(1);
  } else if constexpr (SCHED == 5) {
    // Three-group rotation (see the header comment): twelve wavefronts, three groups of four
    // (one wavefront of each group per SIMD).  Every wavefront runs the same program,
    //   step j = MMA(j) | barrier | SM1(j) | barrier | SM2(j) | barrier,
    // MMA(j) = PV(j-1) + QK(j), SM1 the speculative exponentials, row sum and check (or the
    // plain step), SM2 the 16-bit packing and the rescale of O; group g starts g barriers
    // later.  Between two barriers (a phase) one group issues matrix instructions while the
    // two others are in the two parts of their softmax, so a softmax has two phases to finish
    // and two wavefronts per SIMD issue vector instructions side by side.  With group g's
    // step j in phases 3j+g .. 3j+g+2: K(j) and V(j-1) are read in phases 3j .. 3j+2.  Rings
    // of three slots (tile t in slot t % 3; V slots first, then K slots).  Group 0 issues
    // K(j+2) at the start of phase 3j+1 (into the slot of K(j-1), last read in phase 3j-1)
    // and waits for K(j+1) at the end of phase 3j+2; group 1 issues V(j+1) at the start of
    // phase 3j+2 (into the slot of V(j-2), last read in phase 3j-1) and waits for V(j) at the
    // end of the same phase; each wait is at least one barrier ahead of the tile's first read.
    const int grp = wave >> 2;  // 0, 1, 2
    const int gw = wave & 3;
    using Four = std::integral_constant<int, 4>;
    constexpr int LPT = NCH >= 4 ? NCH / 4 : 1;  // loads per tile of a loading wavefront
    static_assert(NCH % 4 == 0 || 4 % NCH == 0, "tile pieces spread evenly");
    f32x16 S[KB];
    i32x4 P[KS];
    float alpha = 1.f;
    bool rs = false;
    char *const kbase = smem + 3 * TILE;  // K slots; V slots at smem
    for (int t = 0; t < 2; ++t)
      if (t < ntl) load_one(kb_, kbase + t * TILE, jb + t);
    if (ntl > 0) load_one(vb, smem, jb);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    wg_barrier();
    if (grp >= 1) wg_barrier();
    if (grp == 2) wg_barrier();
    // Step j in slot ST = j % 3; phase PH as in schedule 2 (0: QK^T only, 1: PV and QK^T,
    // 2: PV only), the first and last steps outside the loops.
    auto step = [&](auto st_c, auto mask_c, auto ph_c, int j) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr bool MK = decltype(mask_c)::value;
      constexpr int PH = decltype(ph_c)::value;
      constexpr int SP = (ST + 2) % 3;  // slot of tile j - 1 (and of tile j + 2)
      constexpr int SN = (ST + 1) % 3;  // slot of tile j + 1
      if constexpr (PH == 1) {
        pvqk_block<D, BC, F16, 3, SP * TILE, ST * TILE>(smem, P, O[0], kbase, S, qreg[0], ad);
      } else if constexpr (PH == 0) {
        qk_block<D, BC, F16, 3, ST * TILE>(kbase, S, qreg[0], ad);
      } else {
        pv_block<D, BC, F16, 2, SP * TILE>(smem, P, O[0], ad);
      }
      wg_barrier();
      // SM1
      if (grp == 0) {
        if (j + 2 < ntl) load_by(kb_, kbase + SP * TILE, jb + j + 2, gw, Four{});
      } else if (grp == 1) {
        if (j + 1 < ntl) load_by(vb, smem + SN * TILE, jb + j + 1, gw, Four{});
      }
      if constexpr (PH != 2) {
        // (step 0: m is still -inf, the speculation would fail)
        alpha = MK || PH == 0
                    ? softmax_block<BC, F16, MK>(S, P, m[0], l[0], c, MK ? klim[0] - (jb + j) * BC - 4 * hi : 0, rs)
                    : softmax_block_spec<BC, F16>(S, P, m[0], l[0], c, rs);
        lds_dep(l[0]);
      }
      if (grp == 1) {
        // V(j) landed (V(j+1), issued above, may still be in flight)
        if (j + 1 < ntl)
          wait_vmcnt<LPT>();
        else
          wait_vmcnt<0>();
      }
      wg_barrier();
      // SM2: the rescale of O and the pinned 16-bit P~ (left alone, the compiler would sink
      // the conversions into the next matrix phase)
      if constexpr (PH != 2) {
        if (PH != 0 && rs) rescale_o<DT>(O[0], alpha);  // (O is still zero at step 0)
#pragma unroll
        for (int i = 0; i < KS; ++i) lds_dep(P[i]);
      }
      if (grp == 0) {
        // K(j+1) landed; K(j+2), issued in SM1, may still be in flight
        if (j + 2 < ntl)
          wait_vmcnt<LPT>();
        else
          wait_vmcnt<0>();
      }
      wg_barrier();
    };
    const int jm = min(max(kfull[0] - jb, 0), ntl);
    auto run = [&](auto mask_c, int j0, int j1) __attribute__((always_inline)) {
      for (int jj = j0 - j0 % 3; jj < j1; jj += 3) {
        static_for<0, 3>([&](auto st_c) __attribute__((always_inline)) {
          const int j = jj + decltype(st_c)::value;
          if (j >= j0 && j < j1) step(st_c, mask_c, IC<1>{}, j);
        });
      }
    };
    if (ntl > 0) {
      if (jm > 0)
        step(IC<0>{}, std::false_type{}, IC<0>{}, 0);
      else
        step(IC<0>{}, std::true_type{}, IC<0>{}, 0);
      run(std::false_type{}, 1, jm);
      run(std::true_type{}, max(jm, 1), ntl);
      const int sl = ntl % 3;
      if (sl == 0)
        step(IC<0>{}, std::true_type{}, IC<2>{}, ntl);
      else if (sl == 1)
        step(IC<1>{}, std::true_type{}, IC<2>{}, ntl);
      else
        step(IC<2>{}, std::true_type{}, IC<2>{}, ntl);
    }
    // every wavefront passes the same number of barriers
    if (grp <= 1) wg_barrier();
    if (grp == 0) wg_barrier();
    finish(0);
  } else {
    // Ping-pong over two groups of four wavefronts (see the header comment).  Every
    // wavefront runs the same program, step j = MMA(j) | barrier | SM(j) | barrier, where
    // MMA(j) = PV(j-1) + QK(j) and SM(j) is the softmax of tile j; group 1 starts one
    // barrier later, so on each SIMD (one wavefront of each group) one wavefront issues
    // matrix instructions while the other runs its softmax.  K and V tiles each have a
    // 3-slot ring (tile t in slot t % 3; V slots first, then K slots).  With barriers
    // B0, B1, ... and group 0's step j between B(2j) and B(2j+2) (group 1's between B(2j+1)
    // and B(2j+3)): K(j) and V(j-1) are read between B(2j) and B(2j+2).  The loads are
    // issued in the softmax halves only: group 0 issues K(j+2) (into the slot of K(j-1),
    // last read before B(2j)) after B(2j+1) and waits for K(j+1) before B(2j+2); group 1
    // issues V(j+1) (into the slot of V(j-2), last read before B(2j)) after B(2j+2) and waits
    // for it before B(2j+4), at the end of its next matrix half.  Each wait is one barrier
    // ahead of the tile's first read.
    const int grp = wave >> 2;
    const int gw = wave & 3;
    using Four = std::integral_constant<int, 4>;
    constexpr int LPT = NCH >= 4 ? NCH / 4 : 1;  // loads per tile of a loading wavefront
    static_assert(NCH % 4 == 0 || 4 % NCH == 0, "tile pieces spread evenly");
    f32x16 S[KB];
    i32x4 P[KS];
    char *const kbase = smem + 3 * TILE;  // K slots; V slots at smem
    for (int t = 0; t < 2; ++t)
      if (t < ntl) load_one(kb_, kbase + t * TILE, jb + t);
    if (ntl > 0) load_one(vb, smem, jb);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    wg_barrier();
    if (grp == 1) wg_barrier();
    // Step j in slot ST = j % 3 (a compile-time index, so that slot offsets are immediates).
    // Phase PH: 0 for step 0 (QK^T only), 1 for steps 1 .. ntl-1 (PV and QK^T as one MFMA
    // stream), 2 for step ntl (PV only).  The first and last steps run outside the loops, so
    // that the loop body has no branch around its matrix products (with one, the registers
    // of both paths met at the join and the kernel spilled).
    auto step = [&](auto st_c, auto mask_c, auto ph_c, int j) __attribute__((always_inline)) {
      constexpr int ST = decltype(st_c)::value;
      constexpr bool MK = decltype(mask_c)::value;
      constexpr int PH = decltype(ph_c)::value;
      constexpr int SP = (ST + 2) % 3;  // slot of tile j - 1 (and of tile j + 2)
      constexpr int SN = (ST + 1) % 3;  // slot of tile j + 1
      // A slot's offset rides in the reads' 16-bit immediate field when the farthest read of
      // the tile still fits; otherwise (96-key tiles, third slot) the slot goes into the base
      // address and the per-lane addresses are formed again for it.
      constexpr bool VI = SP * TILE + 16 * (KS - 1) * ROWB < 65536;
      constexpr bool KI = ST * TILE + (KB - 1) * 32 * ROWB < 65536;
      constexpr int VO = VI ? SP * TILE : 0, KO = KI ? ST * TILE : 0;
      const char *const vsl = VI ? smem : smem + SP * TILE;
      const char *const ksl = KI ? kbase : kbase + ST * TILE;
      if constexpr (PH == 1) {
        pvqk_block<D, BC, F16, 5, VO, KO>(vsl, P, O[0], ksl, S, qreg[0], ad);
      } else if constexpr (PH == 0) {
        qk_block<D, BC, F16, 6, KO>(ksl, S, qreg[0], ad);
      } else {
        pv_block<D, BC, F16, 4, VO>(vsl, P, O[0], ad);
      }
      if (grp == 1) wait_vmcnt<0>();  // V(j), issued in the previous step, landed
      wg_barrier();
      if (grp == 0) {
        if (j + 2 < ntl) load_by(kb_, kbase + SP * TILE, jb + j + 2, gw, Four{});
      } else {
        if (j + 1 < ntl) load_by(vb, smem + SN * TILE, jb + j + 1, gw, Four{});
      }
      if constexpr (PH != 2) {
        bool rs;
        // (step 0: m is still -inf, so the speculation would fail, and O is still zero, so
        // its rescale by alpha = 0 is left out)
        // (speculation in place: the K tile of this step is still in its slot, so the scores
        // can be formed again if the test fails)
        auto rescore = [&](f32x16(&S2)[KB]) __attribute__((always_inline)) {
          qk_block<D, BC, F16, 6, KO>(ksl, S2, qreg[0], ad);
        };
        const float alpha =
            MK || PH == 0
                ? softmax_block<BC, F16, MK>(S, P, m[0], l[0], c, MK ? klim[0] - (jb + j) * BC - 4 * hi : 0, rs)
                : softmax_block_spec_inplace<BC, F16>(S, P, m[0], l[0], c, rs, rescore);
        if (PH != 0 && rs) rescale_o<DT>(O[0], alpha);
        // The 16-bit P~ and the running sum are formed here, in the softmax half: left to
        // itself the compiler sank their conversions past the barrier, into the start of
        // the next matrix half, ahead of its first LDS reads.
#pragma unroll
        for (int i = 0; i < KS; ++i) lds_dep(P[i]);
        lds_dep(l[0]);
      }
      if (grp == 0) {
        // K(j+1) landed; this step's loads may still be in flight
        if (j + 2 < ntl)
          wait_vmcnt<LPT>();
        else
          wait_vmcnt<0>();
      }
      wg_barrier();
    };
    // Steps [1, jm) take tiles with no masked key, steps [jm, ntl) the others, each range in
    // a loop of its own, as in schedule 0.  With no tile at all (an empty split) there is no
    // step; both groups still pass the same number of barriers.
    const int jm = min(max(kfull[0] - jb, 0), ntl);
    auto run = [&](auto mask_c, int j0, int j1) __attribute__((always_inline)) {
      for (int jj = j0 - j0 % 3; jj < j1; jj += 3) {
        static_for<0, 3>([&](auto st_c) __attribute__((always_inline)) {
          const int j = jj + decltype(st_c)::value;
          if (j >= j0 && j < j1) step(st_c, mask_c, IC<1>{}, j);
        });
      }
    };
    if (ntl > 0) {
      if (jm > 0)
        step(IC<0>{}, std::false_type{}, IC<0>{}, 0);
      else
        step(IC<0>{}, std::true_type{}, IC<0>{}, 0);
      run(std::false_type{}, 1, jm);
      run(std::true_type{}, max(jm, 1), ntl);
      // the last step's slot, ntl % 3, as a compile-time index
      const int sl = ntl % 3;
      if (sl == 0)
        step(IC<0>{}, std::true_type{}, IC<2>{}, ntl);
      else if (sl == 1)
        step(IC<1>{}, std::true_type{}, IC<2>{}, ntl);
      else
        step(IC<2>{}, std::true_type{}, IC<2>{}, ntl);
    }
    if (grp == 0) wg_barrier();
    finish(0);
  }
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16, int SCHED>
hipError_t launch_fa_fwd(const FaArgs &a, hipStream_t stream) {
  FaArgs arg = a;
  void *args[] = {&arg};
  // hipLaunchKernel reports this launch's own status (hipGetLastError would also return a
  // stale error left by some earlier, unrelated runtime call in this thread).
  return hipLaunchKernel((const void *)&fa_fwd_kernel<D, BR, BC, NW, STAGES, F16, SCHED>, dim3(a.total_wgs),
                         dim3(NW * 64), args, 0, stream);
}

template <int D, int BR, int BC, int NW, int STAGES, bool F16, int SCHED = 0>
KernelEntry make_entry() {
  KernelEntry e;
  e.dtype = F16 ? 1 : 0;
  e.d_head = D;
  e.br = BR;
  e.bc = BC;
  e.waves = NW;
  e.stages = STAGES;
  e.schedule = SCHED;
  e.launch = &launch_fa_fwd<D, BR, BC, NW, STAGES, F16, SCHED>;
  e.kernel = (const void *)&fa_fwd_kernel<D, BR, BC, NW, STAGES, F16, SCHED>;
  return e;
}

}  // namespace fa
