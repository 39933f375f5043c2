// fa_bwd_kernel.h -- the gfx950 attention backward pass (device code).
//
// What it computes (page "GPU 内核与 FlashAttention", section 13): given dO, the gradients
// of the forward pass O = softmax(scale Q K^T) V,
//     P = exp(scale Q K^T - L)            (L = the forward's natural-log LSE per row)
//     dV = P^T dO,   dP = dO V^T,   D = rowsum(dO o O),   dS = P o (dP - D),
//     dQ = scale dS K,   dK = scale dS^T Q,
// in the order of that page's blocked backward (section 13.2) and FlashAttention-2's
// parallelisation (section 14.2): one workgroup per (batch, K/V head, tile of BKV keys)
// keeps its keys' dK and dV in registers over the whole loop on query tiles.  With grouped
// K/V heads the loop also runs over every query head of the group, so dK and dV of a K/V
// head are summed on chip (section 14.2).  Under the causal mask the loop starts at the
// first query tile that can see the workgroup's first key, and only tiles crossing the
// diagonal are masked.
//
// dQ is formed one of two ways:
//  * by default, a second, query-parallel pass (fa_bwd_dq_pass_kernel): one workgroup per
//    (batch, head, query tile) recomputes S, P, dP and dS over the key tiles and sums
//    dQ = scale dS K on chip, storing it once (no atomics; bitwise repeatable);
//  * with atomic_dq (the page's Algorithm 2), the dK/dV kernel adds each workgroup's share
//    of dQ into an fp32 accumulator in HBM with atomic adds, converted at the end.
//
// Kernels:
//   fa_bwd_pre_kernel      D_i = <dO_i, O_i> (the page's simplification of P_i . dP_i),
//                          L_i log2(e) for exp2, and (atomic_dq) a zeroed dQ accumulator row;
//   fa_bwd_kernel          the dK/dV loop (and, with atomic_dq, the atomic dQ adds);
//   fa_bwd_dq_pass_kernel  the default dQ pass;
//   fa_bwd_dq_kernel       (atomic_dq) dQ = 16-bit(scale x accumulator).
//
// gfx950 mapping (the forward's building blocks in other roles):
//  * Each wavefront owns 32 keys.  S = Q K^T and dP = dO V^T are formed with the K and V
//    rows of its keys held in registers as the B operand (lane = key) and Q / dO rows read
//    from LDS as the A operand (the forward's qk_block), so in the 32x32 accumulator lane l
//    holds key l%32 and 16 query rows 8g + 4(l/32) + r.
//  * Those registers, P and dS rounded to 16 bits, are directly the B operand of
//    dV^T += dO^T P and dK^T += Q^T dS, whose A operands are read transposed from the
//    row-major dO and Q tiles with ds_read_b64_tr_b16 (the forward's pv_block, with query
//    rows in place of key rows).
//  * atomic_dq: dS also goes to LDS as dS^T [key][query]; after a barrier each wavefront
//    forms two 32x32 tiles of dQ = dS K over all the workgroup's keys, both operands read
//    transposed (dS^T and the resident K tile), and adds them to the accumulator with
//    global atomic adds (no return value).
//  * The dQ pass is the forward's structure with a third product: S^T = K Q^T and
//    dP^T = V dO^T with K, V tiles in LDS and Q, dO in registers, then dQ^T += K^T dS^T
//    with K read transposed.
//  * Q, dO, L log2(e) and D of the next query tile stream into LDS (buffer_load ... lds)
//    while the current one is used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd.h"
#include "fa_fwd_kernel.h"

namespace fa {

// ---------------------------------------------------------------------------------------
// Preprocess: one row (b, i, h) per D/8 lanes, 16-byte loads of O and dO.
template <int D, bool F16>
__global__ void __launch_bounds__(256) fa_bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;      // lanes per row
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
  const int c8 = threadIdx.x % LPR;
  float dot = 0.f;
  const bool valid = row < nq;
  const int64_t elt = ((qrow0 + row) * a.heads + h) * (int64_t)D + 8 * c8;
  if (valid) {
    const i32x4 ov = *(const i32x4 *)((const char *)a.o + elt * 2);
    const i32x4 dv = *(const i32x4 *)((const char *)a.dout + elt * 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // Elements are copied to scalars before __builtin_bit_cast: applied to a vector element
      // directly, this compiler read element 0 in every iteration.
      const int oe = ov[e], de = dv[e];
      f32x2 x, y;
      if constexpr (F16) {
        x = __builtin_convertvector(__builtin_bit_cast(f16x2, oe), f32x2);
        y = __builtin_convertvector(__builtin_bit_cast(f16x2, de), f32x2);
      } else {
        x = __builtin_convertvector(__builtin_bit_cast(bf16x2, oe), f32x2);
        y = __builtin_convertvector(__builtin_bit_cast(bf16x2, de), f32x2);
      }
      dot = __builtin_fmaf(x[0], y[0], dot);
      dot = __builtin_fmaf(x[1], y[1], dot);
    }
    if (a.dq_acc) {  // the atomic path accumulates dQ here
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4 *)(a.dq_acc + elt) = z;
      *(f32x4 *)(a.dq_acc + elt + 4) = z;
    }
  }
  // sum over the LPR lanes of the row (consecutive lanes, LPR a power of two)
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, LPR);
  if (valid && c8 == 0) {
    const int64_t r = ((int64_t)b * a.heads + h) * a.seqlen_q + row;
    a.dvec[r] = dot;
    a.lse2[r] = a.lse[r] * 1.4426950408889634f;
  }
}

// dQ = 16-bit(scale x accumulator), four floats per lane.
template <int D, bool F16>
__global__ void __launch_bounds__(256) fa_bwd_dq_kernel(BwdArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;
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
  const int64_t elt = ((qrow0 + row) * a.heads + h) * (int64_t)D + 4 * c4;
  const f32x4 x = *(const f32x4 *)(a.dq_acc + elt);
  const int lo = pack2<F16>(x[0] * a.scale, x[1] * a.scale);
  const int hi = pack2<F16>(x[2] * a.scale, x[3] * a.scale);
  *(int2 *)((char *)a.dq + elt * 2) = make_int2(lo, hi);
}

// ---------------------------------------------------------------------------------------
// Main kernel.

__device__ __forceinline__ void wait_lds_all() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// dQ tile (32 query rows x 32 d) += dS (32 x BKV keys) K (BKV keys x 32 d), both operands read
// transposed: A from dS^T [key][query] (column = query), B from K [key][d] (column = d).  In a
// 16-key step lane l supplies keys 16 ks + 4(l/32) + {0..3} and 16 ks + 8 + 4(l/32) + {0..3}
// of its column, the order the accumulator layout of the other products uses.
template <int BKV, int AROWB, int BROWB, bool F16, int LA = 3>
__device__ __forceinline__ void dq_block(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x16 &acc) {
  constexpr int N = BKV / 16;
  constexpr int L = LA < N ? LA : N;
  static_assert(4 * L <= 15, "lgkmcnt field");
  i16x4 x0[L + 1], x1[L + 1], y0[L + 1], y1[L + 1];
  auto issue = [&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;  // key step i: rows 16 i + ... of both tiles
    lds_read_tr<16 * i * AROWB>(x0[i % (L + 1)], a0);
    lds_read_tr<16 * i * AROWB>(x1[i % (L + 1)], a1);
    lds_read_tr<16 * i * BROWB>(y0[i % (L + 1)], b0);
    lds_read_tr<16 * i * BROWB>(y1[i % (L + 1)], b1);
  };
  static_for<0, L>(issue);
  static_for<0, N>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    if constexpr (i + L < N) issue(IC<i + L>{});
    constexpr int after = 4 * ((N - 1 - i) < L ? (N - 1 - i) : L);
    lds_wait<after>();
    lds_dep(x0[i % (L + 1)]);
    lds_dep(x1[i % (L + 1)]);
    lds_dep(y0[i % (L + 1)]);
    lds_dep(y1[i % (L + 1)]);
    const i16x4 &p0 = x0[i % (L + 1)], &p1 = x1[i % (L + 1)], &r0 = y0[i % (L + 1)], &r1 = y1[i % (L + 1)];
    const i16x8 av = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    const i16x8 bv = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    acc = mfma32<F16>(__builtin_bit_cast(i32x4, av), __builtin_bit_cast(i32x4, bv), acc);
  });
}

// Store a transposed accumulator tile set (lane = key column l%32, rows d = 32 dt + 8 g +
// 4(l/32) + r) times mul as 16-bit rows of a [rows, heads_kv, D] tensor, as the forward's
// output store does; rows past the buffer's range are dropped.
template <int D, bool F16>
__device__ __forceinline__ void store_rows(const f32x16 (&A)[D / 32], float mul, int row0, uint32_t row_bytes,
                                           const __amdgpu_buffer_rsrc_t &rs, int lane) {
  constexpr int DT = D / 32;
  const int hi = lane >> 5;
  const uint32_t off = (uint32_t)(row0 + (lane & 31)) * row_bytes + hi * 16;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int g0 = 2 * p, g1 = 2 * p + 1;
      const int x0 = pack2<F16>(A[dt][4 * g0 + 0] * mul, A[dt][4 * g0 + 1] * mul);
      const int x1 = pack2<F16>(A[dt][4 * g0 + 2] * mul, A[dt][4 * g0 + 3] * mul);
      const int y0 = pack2<F16>(A[dt][4 * g1 + 0] * mul, A[dt][4 * g1 + 1] * mul);
      const int y1 = pack2<F16>(A[dt][4 * g1 + 2] * mul, A[dt][4 * g1 + 3] * mul);
      auto s0 = __builtin_amdgcn_permlane32_swap((unsigned)x0, (unsigned)y0, false, false);
      auto s1 = __builtin_amdgcn_permlane32_swap((unsigned)x1, (unsigned)y1, false, false);
      const i32x4 out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
      __builtin_amdgcn_raw_buffer_store_b128(out, rs, off + (32 * dt + 16 * p) * 2, 0, 0);
    }
  }
}

// The lane's index within its wavefront, recomputed where it is called (the asm is opaque, so
// values derived from it are neither hoisted out of a loop nor kept live across one).
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// BKV = 32 * NW keys per workgroup, BQ = 64 query rows per step (two 32-row blocks).
// ATOMIC_DQ: also form dQ = dS K here and add it into the fp32 accumulator with atomics (the
// pages' Algorithm 2); otherwise dQ is left to fa_bwd_dq_pass_kernel.
// CAUSAL must equal a.causal.  Without the atomic dQ, keys past the sequence end need no mask:
// each lane's products touch only its own key's dK and dV columns, and those rows are never
// stored (the store goes through a resource bounded by the sequence).
template <int D, int NW, bool F16, bool ATOMIC_DQ, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(ATOMIC_DQ ? 1 : 2)))
fa_bwd_kernel(BwdArgs a) {
  constexpr int BKV = 32 * NW;
  constexpr int BQ = 64;
  constexpr int QB = BQ / 32;        // 32-row query blocks per step
  constexpr int ROWB = D * 2;        // bytes of a Q / dO / K row in LDS
  constexpr int DSROWB = BQ * 2;     // bytes of a dS^T row (one key, BQ queries)
  constexpr int QT = BQ * ROWB;                   // bytes of a Q (or dO) tile
  constexpr int KT = ATOMIC_DQ ? BKV * ROWB : 0;  // bytes of the K tile (dQ product only)
  constexpr int DST = ATOMIC_DQ ? BKV * DSROWB : 0;  // bytes of the dS^T tile (dQ product only)
  constexpr int VT = BQ * 4;         // bytes of an L log2(e) (or D) row segment
  // LDS: K tile | dS^T tile | (Q, dO) x 2 stages | (L log2(e), D) x 2 stages
  constexpr int LDS_BYTES = KT + DST + 4 * QT + 4 * VT;
  constexpr int DT = D / 32;
  constexpr int NCHQ = QT / 1024;    // 1 KB pieces of a Q tile
  constexpr int NCHK = BKV * ROWB / 1024;
  // dQ output tiles of a step: QB x DT, spread over the wavefronts
  constexpr int NTILE = QB * DT;
  constexpr int TPW = NTILE / NW;
  static_assert(NTILE % NW == 0, "dQ tiles per wavefront");
  static_assert(NCHQ % NW == 0 && NCHK % NW == 0, "tile pieces per wavefront");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(D == 32 || D == 64 || D == 128, "d_head");

  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  char *sk = smem;
  char *sds = smem + KT;
  char *sqd = smem + KT + DST;           // stage st: Q at sqd + 2 st QT, dO after it
  char *svec = smem + KT + DST + 4 * QT;  // stage st: L log2(e) at svec + 2 st VT, D after it

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;

  const int w = blockIdx.x;
  const int G = a.total_wgs;
  const int per = G >> 3, rem = G & 7, xcd = w & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  // head-major, as in the forward: every XCD gets a share of every (packed) sequence, and
  // the workgroups of one (sequence, K/V head), which stream the same Q and dO tiles, run
  // together on one XCD.  Under the causal mask the work of a key tile falls with its index;
  // there, within windows of kCausalWindow consecutive (sequence, K/V head) groups, the
  // workgroups go out key tile by key tile (longest first), which evens out the CUs' ends
  // while the window's Q/dO streams still fit the XCD's L2 (windows of 4-8 groups: 2.5-6 %
  // faster; 32: 2 % slower; all groups: 36 % slower).
  constexpr int kCausalWindow = 8;
  int kt = lin % a.n_ktiles;
  int hkb = lin / a.n_ktiles;
  if (CAUSAL) {
    const int ng = a.total_wgs / a.n_ktiles;  // (sequence, K/V head) groups
    const int g0 = hkb - hkb % kCausalWindow;
    const int wg = min(kCausalWindow, ng - g0);
    const int o = lin - g0 * a.n_ktiles;
    kt = o / wg;
    hkb = g0 + o % wg;
  }
  const int b = hkb % a.batch;
  const int hk = hkb / a.batch;

  int nq, nk;
  int64_t qrow0, krow0;
  if (a.cu_seqlens) {
    const int s0 = a.cu_seqlens[b], s1 = a.cu_seqlens[b + 1];
    nq = nk = min(s1 - s0, a.seqlen_q);  // tokens past max_seqlen (a broken contract): not used
    qrow0 = krow0 = s0;
  } else {
    nq = a.seqlen_q;
    nk = a.seqlen_k;
    qrow0 = (int64_t)b * nq;
    krow0 = (int64_t)b * nk;
  }
  const int k0 = kt * BKV;
  if (k0 >= nk || nq <= 0) return;  // uniform over the workgroup

  const int64_t hd = (int64_t)a.heads * D;
  const int64_t hkd = (int64_t)a.heads_kv * D;
  const uint32_t q_row_bytes = (uint32_t)(hd * 2);
  const uint32_t kv_row_bytes = (uint32_t)(hkd * 2);
  const char *kb_ = (const char *)a.k + (krow0 * hkd + (int64_t)hk * D) * 2;
  const char *vb = (const char *)a.v + (krow0 * hkd + (int64_t)hk * D) * 2;
  const auto rk = make_rsrc(kb_, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);
  const auto rv = make_rsrc(vb, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);

  // Tiles to LDS (Q and dO; with the atomic dQ also the K tile, B operand of dQ read
  // transposed), swizzled like the forward's tiles.  Piece u (1 KB) of a tile holds rows
  // RPP u .. RPP u + RPP - 1; lane ln writes row RPP u + ln / CPR, chunk (ln % CPR) XOR
  // swz(row).  A wavefront loads pieces wave, wave + NW, ...; swz looks only at the low four
  // bits of the row, the same for all of them (NW RPP is a multiple of 16), so the lane's
  // part of the global offset is one value and each piece adds a uniform row offset.
  constexpr int RPP = 1024 / ROWB, CPR = ROWB / 16;
  static_assert((NW * RPP) % 16 == 0, "one swizzle pattern per wavefront");
  auto tile_lane_off = [&](uint32_t row_bytes) __attribute__((always_inline)) {
    // the lane id is fetched afresh: offsets recomputed per step cost a few VALU, while
    // offsets kept live across the step loop get spilled, and a reload waits for every
    // load in flight (the prefetch included)
    const uint32_t ln = (uint32_t)fresh_lane_id();
    const int r = wave * RPP + (int)(ln / CPR);
    return (ln / CPR) * row_bytes + (uint32_t)(((int)(ln % CPR) ^ swz<D>(r)) * 16);
  };
  auto load_rows = [&](const __amdgpu_buffer_rsrc_t &rsrc, char *dst, int row0, uint32_t row_bytes, int nch,
                       uint32_t lane_off) __attribute__((always_inline)) {
    for (int u = wave; u < nch; u += NW)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void FA_LDS *)(dst + u * 1024), 16,
                                               (uint32_t)(row0 + u * RPP) * row_bytes + lane_off, 0, 0, 0);
  };
  if constexpr (ATOMIC_DQ) load_rows(rk, sk, k0, kv_row_bytes, NCHK, tile_lane_off(kv_row_bytes));

  // The wavefront's 32 keys in registers: B operand of S = Q K^T (K) and dP = dO V^T (V).
  const int kw0 = k0 + 32 * wave;
  const int my_key = kw0 + (lane & 31);
  i32x4 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const uint32_t off = (uint32_t)my_key * kv_row_bytes + (2 * t + hi) * 16;
    kreg[t] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    vreg[t] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
  }

  f32x16 dKt[DT], dVt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dKt[dt] = f32x16{};
    dVt[dt] = f32x16{};
  }
  const LdsAddr ads = lds_addr<BQ>(lane);  // transposed reads of dS^T (rows of BQ queries)
  const float c = a.scale_log2;

  // Query tiles: all of them, or under the causal mask those holding a row >= k0.
  const int nqt = (nq + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? min(k0 / BQ, nqt) : 0;
  const int nqt_w = nqt - qt0;
  const int n_steps = nqt_w * a.group;  // (query head, query tile) pairs

  // Loads of step s = (head h_of(s), tile qt0 + s % nqt_w) into stage s & 1.
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    const int h = hk * a.group + s / nqt_w;
    const int q0 = (qt0 + s % nqt_w) * BQ;
    char *st = sqd + (s & 1) * 2 * QT;
    char *sv = svec + (s & 1) * 2 * VT;
    const int64_t hoff = (qrow0 * hd + (int64_t)h * D) * 2;
    const auto rq = make_rsrc((const char *)a.q + hoff, (uint32_t)(nq - 1) * q_row_bytes + ROWB);
    const auto rdo = make_rsrc((const char *)a.dout + hoff, (uint32_t)(nq - 1) * q_row_bytes + ROWB);
    const uint32_t lo = tile_lane_off(q_row_bytes);
    load_rows(rq, st, q0, q_row_bytes, NCHQ, lo);
    load_rows(rdo, st + QT, q0, q_row_bytes, NCHQ, lo);
    const int64_t vrow = ((int64_t)b * a.heads + h) * a.seqlen_q;
    if (wave == 0) {
      const auto rl = make_rsrc(a.lse2 + vrow, (uint32_t)nq * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (void FA_LDS *)sv, 4, (uint32_t)(q0 + fresh_lane_id()) * 4, 0, 0, 0);
    } else if (wave == 1) {
      const auto rd = make_rsrc(a.dvec + vrow, (uint32_t)nq * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (void FA_LDS *)(sv + VT), 4, (uint32_t)(q0 + fresh_lane_id()) * 4, 0, 0, 0);
    }
  };

  if (n_steps > 0) issue_step(0);
  // vmcnt bookkeeping: a step's loads are followed (in issue order) only by the next step's
  // loads and by this step's dQ atomics, TPW x 16 per lane.
  constexpr int NATOM = ATOMIC_DQ ? TPW * 16 : 0;
  static_assert(NATOM + 2 * (NCHQ / NW) + 1 <= 63, "vmcnt field");

  // Step s = (query head, query tile) in stage s & 1.
  auto step = [&](int s) __attribute__((always_inline)) {
    // Step s's loads (and, before them, the K tile and registers) have landed once at most
    // the previous step's atomics are still in flight.
    if (s == 0)
      wait_vmcnt<0>();
    else
      wait_vmcnt<NATOM>();
    wg_barrier();  // everyone's loads landed; everyone is done with stage (s+1)&1 and dS^T
    if (s + 1 < n_steps) issue_step(s + 1);

    const int h = hk * a.group + s / nqt_w;
    const int q0 = (qt0 + s % nqt_w) * BQ;
    const char *sq = sqd + (s & 1) * 2 * QT;  // Q of this stage, dO after it
    const int fl = fresh_lane_id();  // per step, for the reason above
    const LdsAddr ad = lds_addr<D>(fl);
    const float *sl2 = (const float *)(svec + (s & 1) * 2 * VT);
    const float *sdv = sl2 + BQ;

    static_for<0, QB>([&](auto qb_c) __attribute__((always_inline)) {
      constexpr int qb = decltype(qb_c)::value;
      constexpr int QO = qb * 32 * ROWB;  // this 32-row block of Q (dO at + QT)
      f32x16 S[1], dP[1];
      // (shorter read lookahead than the forward's: two wavefronts per SIMD hide latency and
      // the registers are needed for dK and dV; S and dP back to back, then P and dS, then
      // the two accumulating products: more independent work than forming dP after dV)
      qk_block<D, 32, F16, 2, QO>(sq, S, kreg, ad);
      qk_block<D, 32, F16, 2, QO + QT>(sq, dP, vreg, ad);
      // rows of this lane: query q0 + 32 qb + 8 g + 4 hi + r; L log2(e) and D are read from
      // LDS four rows at a time, and P and dS packed to 16 bits as they are formed
      const int rb = 32 * qb + 4 * (fl >> 5);
      const int kq = my_key - (q0 + rb);  // (causal) masked where kq > 8 g + r
      i32x4 Pp[2], dSp[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l2 = *(const f32x4 *)(sl2 + rb + 8 * g);
        const f32x4 dd = *(const f32x4 *)(sdv + rb + 8 * g);
        float pv[4], dsv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * g + r;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[0][e], c, -l2[r]));
          // masked: (causal) key past the query; with the atomic dQ also a key past the
          // sequence, whose zero K row would otherwise meet an unbounded P in dS K
          if ((ATOMIC_DQ && my_key >= nk) || (CAUSAL && kq > 8 * g + r)) p = 0.f;
          pv[r] = p;
          dsv[r] = p * (dP[0][e] - dd[r]);
        }
        // register e = 4g + r of step s2 = g / 2, dword (g % 2) * 2 + r / 2
        Pp[g >> 1][2 * (g & 1)] = pack2<F16>(pv[0], pv[1]);
        Pp[g >> 1][2 * (g & 1) + 1] = pack2<F16>(pv[2], pv[3]);
        dSp[g >> 1][2 * (g & 1)] = pack2<F16>(dsv[0], dsv[1]);
        dSp[g >> 1][2 * (g & 1) + 1] = pack2<F16>(dsv[2], dsv[3]);
      }
      pv_block<D, 32, F16, 2, QO + QT>(sq, Pp, dVt, ad);
      // dS^T [key][query] for the dQ product: lane's key row, queries 32 qb + 8 g + 4 hi + 0..3
      if constexpr (ATOMIC_DQ) {
        const int kr = 32 * wave + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * qb + 8 * g + 4 * hi;  // 4 queries = 8 bytes, half a 16-byte chunk
          const int chunk = (col >> 3) ^ swz<BQ>(kr);
          const int2 val = make_int2(dSp[g >> 1][2 * (g & 1)], dSp[g >> 1][2 * (g & 1) + 1]);
          *(int2 *)(sds + kr * DSROWB + chunk * 16 + (col & 7) * 2) = val;
        }
      }
      pv_block<D, 32, F16, 2, QO>(sq, dSp, dKt, ad);
    });
    if constexpr (ATOMIC_DQ) {
    wait_lds_all();
    wg_barrier();  // dS^T complete

    // dQ tiles of this wavefront: tile id = wave * TPW + u -> (query block, d tile).  The
    // adds go through a buffer resource bounding this head's rows below nq, so every lane
    // issues the same number of atomics (rows past the end are dropped by the hardware) and
    // the vmcnt bookkeeping above stays exact.  No cache-policy bits: the same instruction
    // the compiler emits for a device-scope relaxed float atomic add.
    const auto rdq = make_rsrc(a.dq_acc + (qrow0 * a.heads + h) * (int64_t)D,
                               (uint32_t)(nq - 1) * (uint32_t)(hd * 4) + D * 4);
    const uint32_t sk_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sk;
    const uint32_t sds_lds = (uint32_t)(uintptr_t)(const char FA_LDS *)sds;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = wave * TPW + u;
      const int qbt = tile / DT, dt = tile % DT;
      f32x16 acc = f32x16{};
      const uint32_t a0 = sds_lds + (uint32_t)(((64 * qbt) ^ ads.vx0) + ads.vbase0);
      const uint32_t a1 = sds_lds + (uint32_t)(((64 * qbt) ^ ads.vx1) + ads.vbase1);
      const uint32_t b0 = sk_lds + (uint32_t)(((64 * dt) ^ ad.vx0) + ad.vbase0);
      const uint32_t b1 = sk_lds + (uint32_t)(((64 * dt) ^ ad.vx1) + ad.vbase1);
      dq_block<BKV, DSROWB, ROWB, F16>(a0, a1, b0, b1, acc);
      // lane holds d = 32 dt + l%32 of query rows q0 + 32 qbt + 8 g + 4 hi + r
      const uint32_t base = (uint32_t)(q0 + 32 * qbt + 4 * hi) * (uint32_t)(hd * 4) + (32 * dt + (lane & 31)) * 4;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[4 * g + r], rdq,
                                                          base + (uint32_t)(8 * g + r) * (uint32_t)(hd * 4), 0, 0);
    }
    }  // ATOMIC_DQ
  };
  for (int s = 0; s < n_steps; ++s) step(s);

  // dK = scale dS^T Q and dV = P^T dO of this wavefront's 32 keys.
  const auto rdk = make_rsrc((char *)a.dk + (krow0 * hkd + (int64_t)hk * D) * 2, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);
  const auto rdv = make_rsrc((char *)a.dv + (krow0 * hkd + (int64_t)hk * D) * 2, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);
  store_rows<D, F16>(dKt, a.scale, kw0, kv_row_bytes, rdk, lane);
  store_rows<D, F16>(dVt, 1.f, kw0, kv_row_bytes, rdv, lane);
}

// ---------------------------------------------------------------------------------------
// The dQ pass (when dQ is not accumulated with atomics): the forward's structure with query
// rows owned by wavefronts and K/V tiles streamed through LDS, and the products
//     S^T = K Q^T,  dP^T = V dO^T   (K, V rows from LDS; Q, dO in registers, lane = query)
//     P = exp2(S c - L log2 e),  dS = P o (dP - D)   (L, D one value per lane)
//     dQ^T += K^T dS^T              (K read transposed; dS registers as the B operand)
// so dQ is summed over every key on chip and written once: no accumulator, no atomics,
// the same bits on every run.  No running max or rescale: P is final given L.
template <int D, int BC, int NW, bool F16, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
fa_bwd_dq_pass_kernel(BwdArgs a) {
  constexpr int BR = 32 * NW;
  constexpr int ROWB = D * 2;
  constexpr int TILE = BC * ROWB;
  constexpr int NCH = TILE / 1024;
  constexpr int DT = D / 32;
  constexpr int KB = BC / 32;
  constexpr int KS = BC / 16;
  constexpr int STAGE = 2 * TILE;  // K tile then V tile
  constexpr int LPT = 2 * (NCH >= NW ? NCH / NW : 1);
  static_assert(NCH % NW == 0 || NW % NCH == 0, "tile pieces spread evenly");
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;
  const int n_qtiles = (a.seqlen_q + BR - 1) / BR;

  const int w = blockIdx.x;
  const int G = a.batch * a.heads * n_qtiles;
  const int per = G >> 3, rem = G & 7, xcd = w & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  const int qi = lin % n_qtiles;
  const int qt = CAUSAL ? n_qtiles - 1 - qi : qi;
  // (K/V head, sequence, head in group, query tile), as in the forward
  const int ght = lin / n_qtiles;
  const int gi = ght % a.group;
  const int hkb = ght / a.group;
  const int b = hkb % a.batch;
  const int hk = hkb / a.batch;
  const int h = hk * a.group + gi;

  int nq, nk;
  int64_t qrow0, krow0;
  if (a.cu_seqlens) {
    const int s0 = a.cu_seqlens[b], s1 = a.cu_seqlens[b + 1];
    nq = nk = min(s1 - s0, a.seqlen_q);  // tokens past max_seqlen (a broken contract): not used
    qrow0 = krow0 = s0;
  } else {
    nq = a.seqlen_q;
    nk = a.seqlen_k;
    qrow0 = (int64_t)b * nq;
    krow0 = (int64_t)b * nk;
  }
  const int q_tile0 = qt * BR;
  if (q_tile0 >= nq || nk <= 0) return;

  const int64_t hd = (int64_t)a.heads * D;
  const int64_t hkd = (int64_t)a.heads_kv * D;
  const uint32_t row_bytes = (uint32_t)(hd * 2);
  const uint32_t kv_row_bytes = (uint32_t)(hkd * 2);
  const int64_t qoff = (qrow0 * hd + (int64_t)h * D) * 2;
  const auto rq = make_rsrc((const char *)a.q + qoff, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const auto rdo = make_rsrc((const char *)a.dout + qoff, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const auto rdq = make_rsrc((char *)a.dq + qoff, (uint32_t)(nq - 1) * row_bytes + ROWB);
  const int64_t kvoff = (krow0 * hkd + (int64_t)hk * D) * 2;
  const auto rk = make_rsrc((const char *)a.k + kvoff, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);
  const auto rv = make_rsrc((const char *)a.v + kvoff, (uint32_t)(nk - 1) * kv_row_bytes + ROWB);

  const int wrow0 = q_tile0 + wave * 32;
  const int my_row = wrow0 + (lane & 31);
  i32x4 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const uint32_t off = (uint32_t)my_row * row_bytes + (2 * t + hi) * 16;
    qreg[t] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    doreg[t] = __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0);
  }
  // L log2(e) and D of this lane's row (rows past nq: 0, their dQ is not stored)
  const int64_t vrow = ((int64_t)b * a.heads + h) * a.seqlen_q;
  const auto rl = make_rsrc(a.lse2 + vrow, (uint32_t)nq * 4);
  const auto rd = make_rsrc(a.dvec + vrow, (uint32_t)nq * 4);
  // (the b32 load returns the raw bits as an integer)
  const float l2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)my_row * 4, 0, 0));
  const float dd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, (uint32_t)my_row * 4, 0, 0));

  // Tile loads, as in the main kernel: piece u (1 KB) holds rows RPP u .., lane ln writes
  // row RPP u + ln / CPR, chunk (ln % CPR) XOR swz(row); the pieces of a wavefront share the
  // low four row bits, so the lane's part of the offset is one value (the same for the K
  // and V tiles, which have the same row pitch).
  constexpr int RPP = 1024 / ROWB, CPR = ROWB / 16;
  static_assert(NCH <= NW || (NW * RPP) % 16 == 0, "one swizzle pattern per wavefront");
  // (one register, formed once: this pass has registers to spare)
  const uint32_t tile_lane_off = ((uint32_t)lane / CPR) * kv_row_bytes +
                                 (uint32_t)(((lane % CPR) ^ swz<D>(wave * RPP + lane / CPR)) * 16);
  auto load_one = [&](const __amdgpu_buffer_rsrc_t &rsrc, char *dst, int j, uint32_t lane_off)
                      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < (NCH + NW - 1) / NW; ++i) {
      const int u = wave + i * NW;
      if (NCH % NW == 0 || u < NCH)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void FA_LDS *)(dst + u * 1024), 16,
                                                 (uint32_t)(j * BC + u * RPP) * kv_row_bytes + lane_off, 0, 0, 0);
    }
  };

  f32x16 dQt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dQt[dt] = f32x16{};
  const float c = a.scale_log2;
  const LdsAddr ad = lds_addr<D>(lane);
  const int kend = CAUSAL ? min(nk, q_tile0 + BR) : nk;
  const int nkt = (kend + BC - 1) / BC;
  // visible keys of this lane's row: below klim; tiles below kfull need no mask for the
  // wavefront.  (A key past the sequence end is masked too: its zero K row times an unbounded
  // P, when the row's LSE is very negative, is not zero.)
  const int klim = CAUSAL ? min(nk, my_row + 1) : nk;
  const int kfull = (CAUSAL ? min(nk, wrow0 + 1) : nk) / BC;
  const int wave_kend = CAUSAL ? min(nk, wrow0 + 32) : nk;

  auto step = [&](auto st_c, auto mask_c, int j) __attribute__((always_inline)) {
    constexpr int ST = decltype(st_c)::value;
    constexpr bool MK = decltype(mask_c)::value;
    wait_vmcnt<0>();
    wg_barrier();
    if (j + 1 < nkt) {
      constexpr int NS = ST ^ 1;
      load_one(rk, smem + NS * STAGE, j + 1, tile_lane_off);
      load_one(rv, smem + NS * STAGE + TILE, j + 1, tile_lane_off);
    }
    if (!MK || j * BC < wave_kend) {
      f32x16 S[KB], dP[KB];
      // the stage's offset rides in the reads' immediate field
      qk_block<D, BC, F16, 6, ST * STAGE>(smem, S, qreg, ad);
      qk_block<D, BC, F16, 6, ST * STAGE + TILE>(smem, dP, doreg, ad);
      // key of register r in block kb: j BC + 32 kb + 8 (r / 4) + 4 hi + r % 4
      i32x4 dSp[KS];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r], c, -l2));
          if (MK && j * BC + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3) >= klim) p = 0.f;
          dsv[r] = p * (dP[kb][r] - dd);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int e = 0; e < 4; ++e) dSp[2 * kb + s2][e] = pack2<F16>(dsv[8 * s2 + 2 * e], dsv[8 * s2 + 2 * e + 1]);
      }
      pv_block<D, BC, F16, 4, ST * STAGE>(smem, dSp, dQt, ad);
    }
  };
  if (nkt > 0) {
    load_one(rk, smem, 0, tile_lane_off);
    load_one(rv, smem + TILE, 0, tile_lane_off);
  }
  // Tiles [0, jm) need no mask and [jm, nkt) may: each range in a loop of its own (with the
  // mask under a branch the compiler copies the scores between registers on every tile).
  const int jm = min(kfull, nkt);
  auto run = [&](auto mask_c, int j0, int j1) __attribute__((always_inline)) {
    for (int jj = j0 - (j0 & 1); jj < j1; jj += 2) {
      if (jj >= j0) step(IC<0>{}, mask_c, jj);
      if (jj + 1 < j1) step(IC<1>{}, mask_c, jj + 1);
    }
  };
  run(std::false_type{}, 0, jm);
  run(std::true_type{}, jm, nkt);
  (void)LPT;
  store_rows<D, F16>(dQt, a.scale, wrow0, row_bytes, rdq, lane);
}

template <int D, int NW, bool F16, bool ATOMIC_DQ>
hipError_t launch_fa_bwd(const BwdArgs &a, hipStream_t stream) {
  BwdArgs arg = a;
  void *args[] = {&arg};
  constexpr int RPB_PRE = 256 / (D / 8);
  constexpr int RPB_DQ = 256 / (D / 4);
  const int bh = a.batch * a.heads;
  hipError_t e = hipLaunchKernel((const void *)&fa_bwd_pre_kernel<D, F16>,
                                 dim3(bh * ((a.seqlen_q + RPB_PRE - 1) / RPB_PRE)), dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(a.causal ? (const void *)&fa_bwd_kernel<D, NW, F16, ATOMIC_DQ, true>
                               : (const void *)&fa_bwd_kernel<D, NW, F16, ATOMIC_DQ, false>,
                      dim3(a.total_wgs), dim3(NW * 64), args, 0, stream);
  if (e != hipSuccess) return e;
  if constexpr (ATOMIC_DQ) {
    return hipLaunchKernel((const void *)&fa_bwd_dq_kernel<D, F16>, dim3(bh * ((a.seqlen_q + RPB_DQ - 1) / RPB_DQ)),
                           dim3(256), args, 0, stream);
  } else {
    // four wavefronts (128 query rows) per workgroup, two workgroups per CU, whose steps are
    // not tied together by barriers (one eight-wavefront workgroup was 2.7 % slower under the
    // causal mask, the same otherwise); 32-key tiles at d_head 128 keep the pass within 256
    // registers per lane (two wavefronts per SIMD) without spilling
    constexpr int NWQ = 4;
    constexpr int BCQ = D == 128 ? 32 : 64;
    constexpr int BRQ = 32 * NWQ;
    return hipLaunchKernel(a.causal ? (const void *)&fa_bwd_dq_pass_kernel<D, BCQ, NWQ, F16, true>
                                    : (const void *)&fa_bwd_dq_pass_kernel<D, BCQ, NWQ, F16, false>,
                           dim3(bh * ((a.seqlen_q + BRQ - 1) / BRQ)), dim3(NWQ * 64), args, 0, stream);
  }
}

}  // namespace fa
