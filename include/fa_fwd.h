/*
 * fa_fwd.h -- C ABI of an exact-attention forward pass (FlashAttention-2
 * style) for AMD MI355X (gfx950).
 *
 * Operation (page "GPU 内核与 FlashAttention", sections 10, 11 and 14; the
 * kernel interface of "Flash Attention实现深度解析", section 3.1):
 *
 *   for every batch entry b, head h and query row i:
 *     s_ij   = scale * <q[b,i,h,:], k[b,j,h,:]>          (j over the keys)
 *     O[b,i,h,:] = sum_j softmax_j(s_i.) * v[b,j,h,:]
 *     LSE[b,h,i] = log sum_j exp(s_ij)                    (natural log)
 *
 * computed tile by tile with the online softmax, never forming the Nq x Nk
 * score matrix.  Inputs and O are 16-bit (bf16 or fp16, the same type for
 * all four); the softmax and all accumulation are fp32; LSE is fp32.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library allocates no device memory in fa_fwd or fa_fwd_ext and keeps no
 *    pointer after a call returns.
 *  - Dense layout (cu_seqlens == NULL):
 *      q, o : [batch, seqlen_q, n_heads, d_head], contiguous
 *      k, v : [batch, seqlen_k, n_heads, d_head], contiguous
 *      lse  : [batch, n_heads, seqlen_q] fp32
 *  - Packed variable-length layout (cu_seqlens != NULL), self-attention:
 *      cu_seqlens : device int32 [batch + 1], cu[0] = 0, non-decreasing;
 *                   sequence b owns token rows cu[b] .. cu[b+1]-1 of q, k, v, o
 *      q, k, v, o : [cu[batch], n_heads, d_head]
 *      seqlen_q == seqlen_k == the longest sequence length (max_seqlen)
 *      lse        : [batch, n_heads, max_seqlen]; row i of sequence b is
 *                   written only for i < its length, other rows untouched.
 *    The contents of cu_seqlens live on the device and are a precondition
 *    (not checked): they must describe sequences of length <= max_seqlen
 *    inside the q/k/v/o allocations.  A sequence longer than max_seqlen
 *    breaks that contract; the kernels then use only its first max_seqlen
 *    tokens (its later O rows are not written), so LSE writes stay inside
 *    [batch, n_heads, max_seqlen].
 *  - scale is the factor on the raw dot products (1/sqrt(d_head) is usual);
 *    it must be finite and > 0.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without synchronising.
 *  - Argument checks are synchronous, host-only and run before any HIP call;
 *    a call that returns an error has had no effect.  fa_last_error()
 *    returns a message for the calling thread's last non-OK status.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_BF16 = 0, FA_FP16 = 1 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad scale or dtype */
  FA_ERR_UNSUPPORTED = 2, /* d_head not in {32, 64, 128}, sizes past the 32-bit offset limit,
                             or a tile configuration with no compiled kernel */
  FA_ERR_MISALIGNED = 3,  /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_HIP = 4          /* the HIP runtime reported an error (launch, timing, attributes) */
} fa_status_t;

/* A kernel tile configuration (page "Flash Attention 2 Chapter6", the
 * Kernel 7 configuration space: block rows B_r, block columns B_c, warps;
 * the buffering depth of the K/V stream; the instruction schedule).
 *   br       : query rows per workgroup (B_r)
 *   bc       : keys per K/V tile (B_c)
 *   waves    : 64-lane wavefronts per workgroup
 *   stages   : K/V tile pairs resident in LDS (1 = single buffer, 2 = double
 *              buffer, 3-4 = two or three tiles in flight while one is used)
 *   schedule : 0 = each wavefront owns 32 query rows (br = 32 * waves) and runs
 *                  QK^T, softmax and PV of a tile in turn;
 *              1 = each wavefront owns 64 query rows (br = 64 * waves) as two
 *                  32-row blocks whose softmax and matrix products are
 *                  interleaved (one block's softmax runs while the other
 *                  block's products issue; page "GPU 内核与 FlashAttention",
 *                  sections 15.3-15.4); needs stages = 2;
 *              2 = ping-pong: eight wavefronts of 32 rows in two groups that
 *                  alternate, across a workgroup barrier, between the matrix
 *                  products and the softmax (same page, section 15.3); needs
 *                  br = 256, waves = 8 and stages = 3;
 *              4 = schedule 0 with bc = 32 at three wavefronts per SIMD
 *                  (waves = br / 32 of 2 or 4, stages 2 or 3);
 *              5 = three groups of four wavefronts rotating through one
 *                  matrix phase and two softmax phases across workgroup
 *                  barriers; needs br = 384, bc = 32, waves = 12, stages = 3 */
typedef struct {
  int br;
  int bc;
  int waves;
  int stages;
  int schedule;
} fa_tile_config_t;

/* The forward pass.  See the conventions above.  dtype is an fa_dtype_t.
 * Returns an fa_status_t. */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
           int seqlen_q, int seqlen_k, int n_heads, int d_head, float scale,
           const int32_t *cu_seqlens, int dtype, void *stream);

/* Largest num_splits fa_fwd_ext accepts. */
#define FA_MAX_SPLITS 128

/* The forward pass with the options of page "GPU 内核与 FlashAttention",
 * section 14:
 *  - n_heads_kv: K/V heads (MQA/GQA, section 14.2).  It must divide n_heads;
 *    query head h reads K/V head h / (n_heads / n_heads_kv), and nothing is
 *    copied.  k and v are then [batch, seqlen_k, n_heads_kv, d_head] (packed:
 *    [cu[batch], n_heads_kv, d_head]); q, o and lse are as in fa_fwd.
 *    n_heads_kv == n_heads is ordinary multi-head attention.
 *  - causal (0 or 1; section 14.4): the score of key j for query i is -inf
 *    when j > i, with i and j counted from the start of the sequence (so
 *    for seqlen_q != seqlen_k query i sees keys 0..i: top-left aligned).
 *    Key tiles lying wholly above the diagonal are never loaded or computed;
 *    only tiles crossing it are masked element by element.
 *  - num_splits: the keys each query tile visits are divided among this many
 *    workgroups, whose partial results are merged with the (m, l) merge of
 *    section 11.2 by a second kernel on the same stream.  This fills the GPU
 *    when batch x heads x query tiles is small next to the 256 CUs and the
 *    key range is long (a few query rows over many keys).
 *      1            : no split; workspace may be NULL.
 *      2 .. FA_MAX_SPLITS : that many splits; workspace must hold at least
 *                     fa_fwd_workspace_bytes(batch, seqlen_q, n_heads,
 *                     d_head, num_splits) bytes, 16-byte aligned.
 *      0            : automatic: fa_fwd_choose_splits(...), lowered to the
 *                     largest count whose workspace fits workspace_bytes
 *                     (1 if workspace is NULL).
 *    workspace is device memory owned by the caller, used only while the
 *    call's work runs on `stream`; its contents before and after are
 *    irrelevant.  Calls sharing one workspace must be ordered on a stream.
 *    The result equals the unsplit one up to fp32 rounding order.
 * fa_fwd(q, k, v, o, lse, b, nq, nk, h, d, scale, cu, dtype, stream) is
 * fa_fwd_ext(q, k, v, o, lse, b, nq, nk, h, h, d, scale, 0, cu, dtype, 1,
 * NULL, 0, stream).  Returns an fa_status_t. */
int fa_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
               int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale,
               int causal, const int32_t *cu_seqlens, int dtype, int num_splits, void *workspace,
               size_t workspace_bytes, void *stream);

/* Bytes of workspace fa_fwd_ext needs for num_splits splits:
 * num_splits x batch x n_heads x seqlen_q x (d_head + 1) x 4 (each split's
 * fp32 output rows and natural-log LSE; packed layout: seqlen_q is the
 * longest length).  0 for num_splits == 1, and 0 with fa_last_error() set
 * on bad arguments.  Host-only. */
size_t fa_fwd_workspace_bytes(int batch, int seqlen_q, int n_heads, int d_head, int num_splits);

/* The split count num_splits = 0 resolves to before the workspace limit:
 * 1 when batch x n_heads x query tiles already gives every CU work, else
 * enough splits for about two workgroups per CU, at most one per four key
 * tiles and at most FA_MAX_SPLITS.  causal and varlen are 0 or 1.
 * Host-only; < 0 on bad arguments. */
int fa_fwd_choose_splits(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype,
                         int causal, int varlen);

/* Bytes of the device array fa_fwd_ext_noalloc takes its split scratch from (16 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* fa_fwd_ext for callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments, layouts, results and
 * errors as fa_fwd_ext, without the workspace: a split call's scratch (the per-split fp32
 * partial outputs and LSE rows) is a library-owned device array of FA_NOALLOC_SCRATCH_BYTES
 * per GPU, held from library load until the process ends.  The call allocates nothing and
 * calls no allocating routine.
 *  - num_splits > 1 needing more than FA_NOALLOC_SCRATCH_BYTES
 *    (fa_fwd_workspace_bytes(...) > it) -> FA_ERR_INVALID_ARG with a message naming both
 *    sizes; num_splits = 0 lowers the automatic count to what the array holds.
 *  - All calls on one GPU share its array and it keeps the last call's contents (nothing in
 *    it has to start at zero).  Calls that overlap in time on one GPU race on it: issue them
 *    on one stream, or serialise them.
 *  - The first call on a device resolves the array's device address (hipGetSymbolAddress,
 *    with that device current); a failure there -> FA_ERR_HIP. */
int fa_fwd_ext_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                       int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale,
                       int causal, const int32_t *cu_seqlens, int dtype, int num_splits, void *stream);

/* Backward pass (page "GPU 内核与 FlashAttention", section 13; FlashAttention-2's
 * parallelisation over K/V tiles, section 14.2).  Given the forward's inputs,
 * its output o and natural-log lse (from fa_fwd or fa_fwd_ext with the same
 * arguments) and dout = dPhi/dO, writes
 *   dq = dPhi/dq, dk = dPhi/dk, dv = dPhi/dv
 * with P = exp(scale q k^T - lse), dV = P^T dO, dP = dO V^T,
 * D = rowsum(dO o O), dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * Layouts, n_heads_kv, causal and cu_seqlens as in fa_fwd_ext: dout, dq like
 * q; dk, dv like k.  With grouped K/V heads dk and dv of a K/V head sum the
 * contributions of all its query heads.  16-bit outputs are rounded once
 * from fp32.
 * atomic_dq selects how dQ is formed:
 *   0: a second pass over query tiles recomputes S, P, dP and dS and sums
 *      dQ on chip (no atomics; the same bits on every run);
 *   1: the pages' Algorithm 2: the K/V-tile pass adds its share of dQ into
 *      an fp32 accumulator in the workspace with atomic adds (dQ's last bit
 *      may then vary from run to run).
 * workspace: device memory of at least fa_bwd_workspace_bytes(batch,
 * seqlen_q, n_heads, d_head, atomic_dq) bytes, 16-byte aligned,
 * caller-owned; contents irrelevant before and after.  Enqueued on `stream`
 * (three kernels).  Argument checks as in fa_fwd_ext, plus non-null o, dout,
 * dq, dk, dv (16-byte aligned) and workspace; atomic_dq must be 0 or 1.
 * Returns an fa_status_t. */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, int batch, int seqlen_q, int seqlen_k,
           int n_heads, int n_heads_kv, int d_head, float scale, int causal,
           const int32_t *cu_seqlens, int dtype, int atomic_dq, void *workspace,
           size_t workspace_bytes, void *stream);

/* Workspace bytes fa_bwd needs: batch x seqlen_q x n_heads x 2 x 4 (D and
 * L log2(e) per query row), plus batch x seqlen_q x n_heads x d_head x 4 for
 * the fp32 dQ accumulator when atomic_dq is 1 (packed layout: seqlen_q is
 * the longest length).  0 with fa_last_error() set on bad arguments.
 * Host-only. */
size_t fa_bwd_workspace_bytes(int batch, int seqlen_q, int n_heads, int d_head, int atomic_dq);

/* Tile autotuner (page "Flash Attention 2 Chapter6", Kernel 7: enumerate the
 * configuration space, drop configurations that spill registers or do not
 * fit, time the rest, keep the best).  The space is every compiled
 * configuration of (dtype, d_head): B_r in {64, 128, 256} x B_c in
 * {32, 64, 128} x wavefronts x K/V stages x schedule, less those over the
 * 160 KB LDS budget or that spill (fa_fwd_num_configs / fa_fwd_list_configs
 * list it).  Arguments and checks are fa_fwd_ext's; the call's kind --
 * n_heads_kv, causal, packed or dense, num_splits (0 = each candidate's
 * automatic count, lowered to what workspace holds) -- is tuned as given, on
 * the caller's buffers and stream.
 *
 * Timing: the default configuration is launched for about 40 ms first, so
 * the clock reaches its loaded state; then `rounds` (1 .. 100) interleaved
 * rounds each time every candidate once (enough launches per sample for
 * about 0.5 ms), the order rotating by one per round; a candidate's score is
 * its median time per launch.  The two best are then timed against each
 * other for 2 x rounds more rounds, alternating which goes first, and the
 * faster median wins.
 *
 * The winner is remembered for calls of the same kind and size class:
 * (d_head, dtype, packed, causal, ceil(log2(n_heads / n_heads_kv)),
 * ceil(log2 seqlen_q), ceil(log2(batch x n_heads))), and fa_fwd / fa_fwd_ext
 * use it unless a forced configuration applies (fa_fwd_set_config,
 * FA_FWD_CONFIG).  When the environment variable FA_FWD_TUNE_CACHE names a
 * file, the remembered choices are read from it at the first configuration
 * lookup and the file is rewritten after every tuning (FA_ERR_INVALID_ARG,
 * with the choice still remembered, if it cannot be written).
 * O and LSE are overwritten; the last launch uses the winner, so they hold
 * its result.  Synchronises `stream`.  chosen and best_ms (either may be
 * NULL) receive the winner and its median time per launch in ms.  A failed
 * HIP call (launch, event) returns FA_ERR_HIP. */
int fa_fwd_autotune_ext(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                        int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale,
                        int causal, const int32_t *cu_seqlens, int dtype, int num_splits, void *workspace,
                        size_t workspace_bytes, void *stream, int rounds, fa_tile_config_t *chosen,
                        float *best_ms);

/* fa_fwd_autotune_ext for an fa_fwd call: n_heads_kv = n_heads, causal 0,
 * no split; `reps` is the number of rounds. */
int fa_fwd_autotune(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                    int seqlen_q, int seqlen_k, int n_heads, int d_head, float scale,
                    const int32_t *cu_seqlens, int dtype, void *stream, int reps,
                    fa_tile_config_t *chosen, float *best_ms);

/* The last tuning's candidates, fastest first (the two best with their
 * head-to-head medians): copies up to `capacity` configurations and median
 * ms per launch; returns how many there were (0 before any tuning; < 0 on
 * bad arguments).  Host-only. */
int fa_fwd_tune_ranking(fa_tile_config_t *cfgs, float *ms, int capacity);

/* Forget every remembered tuning result (the cache file is left alone).  Host-only. */
int fa_fwd_tune_reset(void);

/* Write the remembered tuning results to `path` in the FA_FWD_TUNE_CACHE
 * format (one line per choice).  FA_ERR_INVALID_ARG if it cannot be written.
 * Host-only. */
int fa_fwd_tune_save(const char *path);

/* Merge tuning results from a file in that format; lines for configurations
 * this build lacks are skipped.  Returns the number of choices taken, or
 * -FA_ERR_INVALID_ARG if the file cannot be read.  Host-only. */
int fa_fwd_tune_load(const char *path);

/* Force the configuration fa_fwd uses for (d_head, dtype); cfg == NULL
 * returns to automatic choice.  Automatic choice, in order: the environment
 * variable FA_FWD_CONFIG="br,bc,waves,stages,schedule" (read once; applies
 * to every (d_head, dtype) that has that configuration compiled), then a
 * configuration the autotuner chose for this call's kind and size class,
 * then the built-in default.  FA_ERR_UNSUPPORTED if no kernel was compiled for cfg. */
int fa_fwd_set_config(int d_head, int dtype, const fa_tile_config_t *cfg);

/* The configuration fa_fwd would use for this shape (host-only lookup).
 * varlen is 0 or 1. */
int fa_fwd_get_config(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype,
                      int varlen, fa_tile_config_t *out);

/* As fa_fwd_get_config, for a call of fa_fwd_ext with this causal flag (0 or 1): the
 * configuration fa_fwd_ext would use (host-only lookup). */
int fa_fwd_get_config_ext(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype,
                          int varlen, int causal, fa_tile_config_t *out);

/* The configuration and automatic split count fa_fwd_ext would use for a call
 * of this shape and kind (varlen, causal 0 or 1; n_heads_kv divides n_heads),
 * and where the configuration comes from: *source = 0 the built-in default,
 * 1 a tuned choice, 2 FA_FWD_CONFIG, 3 fa_fwd_set_config.  num_splits and
 * source may be NULL; the split count is before lowering to a workspace.
 * Host-only lookup. */
int fa_fwd_query_config(int batch, int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head,
                        int dtype, int varlen, int causal, fa_tile_config_t *out, int *num_splits,
                        int *source);

/* Number of compiled configurations for (d_head, dtype); < 0 on bad args. */
int fa_fwd_num_configs(int d_head, int dtype);

/* Copies up to `capacity` compiled configurations for (d_head, dtype) into
 * out; returns how many there are in total (< 0 on bad args).  Host-only. */
int fa_fwd_list_configs(int d_head, int dtype, fa_tile_config_t *out, int capacity);

/* LDS bytes a configuration uses per workgroup, from the configuration alone:
 * stages x (K tile + V tile) for schedule 0, five tiles (two K, three V) for
 * schedule 1; a tile is bc x d_head 16-bit values.  Host-only; < 0 on bad args. */
int fa_fwd_config_lds_bytes(int d_head, const fa_tile_config_t *cfg);

/* Register and spill figures the compiler reports for a compiled
 * configuration (hipFuncGetAttributes): vector registers per lane
 * (architectural + accumulation), private (spill) bytes per lane, static LDS
 * bytes.  Any output pointer may be NULL.  Needs the HIP runtime (a GPU). */
int fa_fwd_config_resources(int d_head, int dtype, const fa_tile_config_t *cfg, int *vgprs,
                            int *spill_bytes, int *lds_bytes);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *fa_last_error(void);

/* Library version string. */
const char *fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
