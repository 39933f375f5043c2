// fa_fwd_api.cpp -- the C ABI declared in include/fa_fwd.h: argument checks, the registry
// of compiled tile configurations, configuration choice, launch, and the autotuner.
//
// Argument checks run on the host before any HIP call, so a rejected call touches
// neither the device nor the runtime.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "fa_bwd.h"
#include "fa_fwd.h"
#include "fa_internal.h"

namespace {

using fa::FaArgs;
using fa::KernelEntry;

thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
  g_last_error = msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return FA_OK;
}

// ---------------------------------------------------------------- registry
std::vector<KernelEntry> *g_entries = nullptr;

void add_entry(const KernelEntry &e) { g_entries->push_back(e); }

template <int D, bool F16, int P = 0>
void register_all() {
  if constexpr (P < fa::kSpaceParts) {
    fa::register_part<D, F16, P>(add_entry);
    register_all<D, F16, P + 1>();
  }
}

const std::vector<KernelEntry> &entries() {
  static std::once_flag once;
  std::call_once(once, [] {
    g_entries = new std::vector<KernelEntry>();
    register_all<32, false>();
    register_all<64, false>();
    register_all<128, false>();
    register_all<32, true>();
    register_all<64, true>();
    register_all<128, true>();
  });
  return *g_entries;
}

const KernelEntry *find_entry(int dtype, int d, const fa_tile_config_t &c) {
  for (const auto &e : entries())
    if (e.dtype == dtype && e.d_head == d && e.br == c.br && e.bc == c.bc && e.waves == c.waves &&
        e.stages == c.stages && e.schedule == c.schedule)
      return &e;
  return nullptr;
}

fa_tile_config_t cfg_of(const KernelEntry &e) { return fa_tile_config_t{e.br, e.bc, e.waves, e.stages, e.schedule}; }

bool valid_dtype(int dtype) { return dtype == FA_BF16 || dtype == FA_FP16; }
bool valid_d(int d) { return d == 32 || d == 64 || d == 128; }

// ------------------------------------------------------ configuration choice
std::mutex g_cfg_mu;
std::map<std::pair<int, int>, fa_tile_config_t> g_forced;  // (d, dtype) -> config

// What a call's configuration choice depends on.
struct Shape {
  int batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d, dtype;
  bool varlen, causal;
};

int log2_bucket(int64_t n) {
  int b = 0;
  while ((int64_t(1) << b) < n) ++b;
  return b;
}

// A tuned choice serves calls of the same kind and about the same size: (d_head, dtype,
// varlen, causal, ceil(log2 of the query heads per K/V head), ceil(log2 seqlen_q),
// ceil(log2 batch x n_heads)).
typedef std::array<int, 7> TuneKey;
TuneKey key_of(const Shape &s) {
  return TuneKey{s.d, s.dtype, s.varlen ? 1 : 0, s.causal ? 1 : 0, log2_bucket(s.n_heads / s.n_heads_kv),
                 log2_bucket(s.seqlen_q), log2_bucket((int64_t)s.batch * s.n_heads)};
}
struct Tuned {
  fa_tile_config_t cfg;
  float ms;  // the winner's median time per launch when it was tuned
};
std::map<TuneKey, Tuned> g_tuned;

// Built-in choice, from sweeps of the compiled configurations on MI355X: a short query
// tile gains nothing from more wavefronts; at d_head 128 and longer sequences eight
// wavefronts sharing one K/V stream per CU are fastest, except under the causal mask (below);
// otherwise two workgroups of four.
fa_tile_config_t default_config(int seqlen_q, int d, bool causal) {
  if (seqlen_q <= 64) return fa_tile_config_t{64, 64, 2, 2, 0};
  if (d == 128 && seqlen_q > 128) {
    // Under the causal mask half the key tiles are skipped and the diagonal ones are short;
    // three four-wavefront workgroups per CU (32-key tiles) then hide more of each step's
    // latency than the eight-wavefront tile does (about 7% on B16 N4096 H16).
    if (causal) return fa_tile_config_t{128, 32, 4, 2, 4};
    // Eight wavefronts in the ping-pong schedule: each SIMD's two wavefronts alternate matrix
    // and softmax halves (3-5% over schedule 0 on full, gqa and varlen).
    return fa_tile_config_t{256, 64, 8, 3, 2};
  }
  return fa_tile_config_t{128, 64, 4, 2, 0};
}

// FA_FWD_CONFIG="br,bc,waves,stages,schedule" in the environment forces that configuration
// for every (d_head, dtype) that has it compiled (read once, at the first configuration
// lookup; fa_fwd_set_config still overrides it).
const fa_tile_config_t *env_config() {
  static fa_tile_config_t cfg;
  static bool have = false;
  static std::once_flag once;
  std::call_once(once, [] {
    const char *e = std::getenv("FA_FWD_CONFIG");
    if (e && std::sscanf(e, "%d,%d,%d,%d,%d", &cfg.br, &cfg.bc, &cfg.waves, &cfg.stages, &cfg.schedule) == 5)
      have = true;
  });
  return have ? &cfg : nullptr;
}

// ------------------------------------------------------------ tuned-choice cache file
// One line per tuned choice:
//   d_head dtype varlen causal log2_group log2_seqlen_q log2_batch_heads : br bc waves stages schedule ms
// Lines starting with '#', malformed lines and configurations this build does not have are
// skipped on reading.
const char *kCacheHeader =
    "# fa_fwd tuned tile configurations: d_head dtype varlen causal log2_group log2_seqlen_q "
    "log2_batch_heads : br bc waves stages schedule ms";

// Caller holds g_cfg_mu.  Returns the number of entries taken, or -1 if the file cannot be read.
int load_cache_locked(const char *path) {
  FILE *f = std::fopen(path, "r");
  if (!f) return -1;
  char line[512];
  int n = 0;
  while (std::fgets(line, sizeof line, f)) {
    if (line[0] == '#') continue;
    TuneKey k;
    fa_tile_config_t c;
    float ms = 0.f;
    if (std::sscanf(line, "%d %d %d %d %d %d %d : %d %d %d %d %d %f", &k[0], &k[1], &k[2], &k[3], &k[4], &k[5],
                    &k[6], &c.br, &c.bc, &c.waves, &c.stages, &c.schedule, &ms) != 13)
      continue;
    if (!find_entry(k[1], k[0], c)) continue;
    g_tuned[k] = Tuned{c, ms};
    ++n;
  }
  std::fclose(f);
  return n;
}

// Caller holds g_cfg_mu.  Writes the whole table (through a temporary file, renamed into place).
int save_cache_locked(const char *path) {
  const std::string tmp = std::string(path) + ".tmp";
  FILE *f = std::fopen(tmp.c_str(), "w");
  if (!f) return -1;
  std::fprintf(f, "%s\n", kCacheHeader);
  for (const auto &kv : g_tuned) {
    const TuneKey &k = kv.first;
    const fa_tile_config_t &c = kv.second.cfg;
    std::fprintf(f, "%d %d %d %d %d %d %d : %d %d %d %d %d %.5f\n", k[0], k[1], k[2], k[3], k[4], k[5], k[6], c.br,
                 c.bc, c.waves, c.stages, c.schedule, kv.second.ms);
  }
  const bool good = std::fclose(f) == 0;
  if (!good || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return -1;
  }
  return 0;
}

// FA_FWD_TUNE_CACHE names a cache file: read at the first configuration lookup, rewritten
// after each tuning.
const char *cache_path() {
  const char *p = std::getenv("FA_FWD_TUNE_CACHE");
  return (p && *p) ? p : nullptr;
}

void load_env_cache_once() {
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char *p = cache_path()) {
      std::lock_guard<std::mutex> lk(g_cfg_mu);
      (void)load_cache_locked(p);
    }
  });
}

// Where a configuration choice came from (fa_fwd_query_config's source).
enum { kSrcDefault = 0, kSrcTuned = 1, kSrcEnv = 2, kSrcForced = 3 };

fa_tile_config_t choose_config(const Shape &s, int *source = nullptr) {
  load_env_cache_once();
  const fa_tile_config_t *env = env_config();
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  int src = kSrcDefault;
  fa_tile_config_t c;
  auto f = g_forced.find({s.d, s.dtype});
  auto t = g_tuned.find(key_of(s));
  if (f != g_forced.end()) {
    c = f->second;
    src = kSrcForced;
  } else if (env && find_entry(s.dtype, s.d, *env)) {
    c = *env;
    src = kSrcEnv;
  } else if (t != g_tuned.end()) {
    c = t->second.cfg;
    src = kSrcTuned;
  } else {
    c = default_config(s.seqlen_q, s.d, s.causal);
  }
  if (source) *source = src;
  return c;
}

// ------------------------------------------------------------ arg checks
int check_args(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
               int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale,
               int causal, const int32_t *cu_seqlens, int dtype) {
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o and lse must be non-null device pointers");
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (batch < 1 || n_heads < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(FA_ERR_INVALID_ARG, "batch, n_heads, seqlen_q and seqlen_k must be >= 1");
  if (n_heads_kv < 1 || n_heads % n_heads_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "n_heads_kv must be >= 1 and divide n_heads");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!valid_d(d_head)) return fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  if (cu_seqlens && seqlen_q != seqlen_k)
    return fail(FA_ERR_INVALID_ARG, "with cu_seqlens, seqlen_q and seqlen_k must both be the max length");
  auto mis = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; };
  if (mis(q, 16) || mis(k, 16) || mis(v, 16) || mis(o, 16))
    return fail(FA_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if (mis(lse, 4)) return fail(FA_ERR_MISALIGNED, "lse must be 4-byte aligned");
  // Per-sequence byte offsets are 32-bit in the kernel (buffer addressing); one tile of
  // slack past the longest sequence.  The fp32 split partials of one (split, batch, head)
  // hold seqlen_q x d_head x 4 bytes.
  const int64_t row_bytes = (int64_t)n_heads * d_head * 2;
  const int64_t longest = std::max(seqlen_q, seqlen_k);
  if ((longest + 256) * row_bytes >= (int64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "sequence length x n_heads x d_head too large for 32-bit offsets");
  const int64_t wgs = (int64_t)batch * n_heads * ((seqlen_q + 63) / 64) * FA_MAX_SPLITS;
  if (wgs >= (int64_t)INT32_MAX) return fail(FA_ERR_UNSUPPORTED, "grid too large");
  return FA_OK;
}

FaArgs make_args(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                 int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, float scale, int causal,
                 const int32_t *cu_seqlens, int br, int num_splits, float *o_part, float *lse_part) {
  FaArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.seqlen_q = seqlen_q;
  a.seqlen_k = seqlen_k;
  a.heads = n_heads;
  a.heads_kv = n_heads_kv;
  a.group = n_heads / n_heads_kv;
  a.causal = causal;
  a.num_splits = num_splits;
  a.n_qtiles = (seqlen_q + br - 1) / br;
  a.total_wgs = batch * n_heads * a.n_qtiles * num_splits;
  a.div_splits = fa::make_fastdiv((uint32_t)num_splits);
  a.div_qtiles = fa::make_fastdiv((uint32_t)a.n_qtiles);
  a.div_group = fa::make_fastdiv((uint32_t)a.group);
  a.div_heads_kv = fa::make_fastdiv((uint32_t)n_heads_kv);
  a.div_batch = fa::make_fastdiv((uint32_t)batch);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
  a.o_part = o_part;
  a.lse_part = lse_part;
  return a;
}

// One forward call on a resolved configuration and split count.  Split mode puts the fp32
// partial outputs at the start of the workspace and their LSE rows after them.
struct Call {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head;
  float scale;
  int causal;
  const int32_t *cu_seqlens;
  int dtype;
  void *stream;
};

size_t workspace_bytes_of(int batch, int seqlen_q, int n_heads, int d_head, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)num_splits * (size_t)batch * (size_t)n_heads * (size_t)seqlen_q * (size_t)(d_head + 1) * 4u;
}

int launch_entry(const KernelEntry &e, const Call &c, int num_splits, void *workspace) {
  float *o_part = nullptr, *lse_part = nullptr;
  if (num_splits > 1) {
    o_part = static_cast<float *>(workspace);
    lse_part = o_part + (size_t)num_splits * c.batch * c.n_heads * c.seqlen_q * c.d_head;
  }
  const FaArgs a = make_args(c.q, c.k, c.v, c.o, c.lse, c.batch, c.seqlen_q, c.seqlen_k, c.n_heads,
                             c.n_heads_kv, c.scale, c.causal, c.cu_seqlens, e.br, num_splits, o_part,
                             lse_part);
  hipStream_t s = reinterpret_cast<hipStream_t>(c.stream);
  hipError_t err = e.launch(a, s);
  if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(err));
  if (num_splits > 1) {
    fa::MergeArgs m;
    m.o_part = o_part;
    m.lse_part = lse_part;
    m.o = c.o;
    m.lse = c.lse;
    m.cu_seqlens = c.cu_seqlens;
    m.batch = c.batch;
    m.seqlen_q = c.seqlen_q;
    m.heads = c.n_heads;
    m.num_splits = num_splits;
    err = fa::launch_merge(m, c.d_head, c.dtype, s);
    if (err != hipSuccess)
      return fail(FA_ERR_HIP, std::string("merge kernel launch failed: ") + hipGetErrorString(err));
  }
  return ok();
}

int launch_entry(const KernelEntry &e, const Call &c) { return launch_entry(e, c, 1, nullptr); }

Call make_call(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
               int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale, int causal,
               const int32_t *cu_seqlens, int dtype, void *stream) {
  return Call{q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale, causal,
              cu_seqlens, dtype, stream};
}

constexpr int kNumCUs = 256;

// Splits for about two workgroups per CU when configuration c's grid alone is smaller than
// the CU count; each split keeps at least four key tiles (measured on MI355X over a few query
// rows against 2K-32K keys: fewer tiles per split cost more in partial stores and merging
// than the extra parallelism gains).
int splits_for(const fa_tile_config_t &c, const Shape &s) {
  const int64_t wgs = (int64_t)s.batch * s.n_heads * ((s.seqlen_q + c.br - 1) / c.br);
  if (wgs >= kNumCUs) return 1;
  const int64_t keys = s.causal ? std::min(s.seqlen_k, s.seqlen_q) : s.seqlen_k;
  const int64_t nkt = (keys + c.bc - 1) / c.bc;
  int64_t n = (2 * kNumCUs + wgs - 1) / wgs;
  n = std::min<int64_t>(n, nkt / 4);
  n = std::min<int64_t>(n, FA_MAX_SPLITS);
  return (int)std::max<int64_t>(n, 1);
}

// The automatic count for c, lowered to the largest one whose partials fit the workspace.
int splits_within(const fa_tile_config_t &c, const Shape &s, const void *workspace, size_t workspace_bytes) {
  int n = splits_for(c, s);
  while (n > 1 && (!workspace || workspace_bytes_of(s.batch, s.seqlen_q, s.n_heads, s.d, n) > workspace_bytes)) --n;
  return n;
}

constexpr int kLdsLimit = 160 * 1024;

// K and V tiles resident in LDS: stages (K, V) pairs for schedules 0 and 2; a 2-slot K ring
// plus a 3-slot V ring for schedule 1.
int lds_bytes_of(int d, const fa_tile_config_t &c) {
  const int tile = c.bc * d * 2;
  return c.schedule == 1 ? 5 * tile : c.stages * 2 * tile;
}

// Backward workspace: D and L log2(e) per query row, and the fp32 dQ accumulator when dQ is
// formed with atomic adds.
size_t bwd_bytes(int batch, int seqlen_q, int n_heads, int d_head, int atomic_dq) {
  return (size_t)batch * (size_t)seqlen_q * (size_t)n_heads * (size_t)((atomic_dq ? d_head : 0) + 2) * 4u;
}

// ------------------------------------------------------------ autotuner
// Page "Flash Attention 2 Chapter6", Kernel 7: enumerate the configuration space, filter
// what cannot run (LDS, spills), time the rest on the caller's buffers, keep the best.
// Timing is made fair to every candidate: the clock is first brought to its loaded state
// (a sequential sweep that starts cold favours whatever runs last: 12-20 % errors were seen
// on MI355X), then all candidates are timed in interleaved rounds with a rotating order and
// scored by their median, and the two best are timed against each other once more.
constexpr int kMaxTuneRounds = 100;
constexpr float kWarmMs = 40.f;    // GPU time spent warming up before any measurement
constexpr float kSampleMs = 0.5f;  // launches per measurement: enough for about this long

std::mutex g_tune_mu;  // one tuning at a time; guards g_last_ranking
struct Candidate {
  const KernelEntry *e = nullptr;
  int splits = 1;
  float ms = 0.f;  // median time per launch
};
struct Ranked {
  fa_tile_config_t cfg;
  float ms;
};
std::vector<Ranked> g_last_ranking;  // the last tuning's candidates, fastest first

float median_of(std::vector<float> v) {
  std::sort(v.begin(), v.end());
  const size_t n = v.size();
  return n % 2 ? v[n / 2] : 0.5f * (v[n / 2 - 1] + v[n / 2]);
}

// Owns a set of HIP events.
struct Events {
  std::vector<hipEvent_t> ev;
  ~Events() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  int create(size_t n) {
    ev.assign(n, nullptr);
    for (auto &e : ev) {
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("hipEventCreate: ") + hipGetErrorString(err));
    }
    return FA_OK;
  }
};

int hip_status(hipError_t err, const char *what) {
  return err == hipSuccess ? FA_OK : fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
}

// ms between two recorded events (the second already complete).
int elapsed(hipEvent_t a, hipEvent_t b, float *ms) { return hip_status(hipEventElapsedTime(ms, a, b), "hipEventElapsedTime"); }

int tune(const Call &call, const Shape &shape, int num_splits, void *workspace, size_t workspace_bytes, int rounds,
         Candidate *best) {
  hipStream_t s = reinterpret_cast<hipStream_t>(call.stream);
  std::vector<Candidate> cand;
  const fa_tile_config_t dflt = default_config(shape.seqlen_q, shape.d, shape.causal);
  size_t first = 0;
  for (const auto &e : entries()) {
    if (e.dtype != shape.dtype || e.d_head != shape.d) continue;
    const fa_tile_config_t c = cfg_of(e);
    if (lds_bytes_of(shape.d, c) > kLdsLimit) continue;  // does not fit one CU's LDS
    hipFuncAttributes attr;
    int st = hip_status(hipFuncGetAttributes(&attr, e.kernel), "hipFuncGetAttributes");
    if (st != FA_OK) return st;
    if (attr.localSizeBytes > 0) continue;  // spills registers
    Candidate cd;
    cd.e = &e;
    cd.splits = num_splits == 0 ? splits_within(c, shape, workspace, workspace_bytes) : num_splits;
    if (std::memcmp(&c, &dflt, sizeof c) == 0) first = cand.size();
    cand.push_back(cd);
  }
  if (cand.empty()) return fail(FA_ERR_UNSUPPORTED, "no compiled configuration passed the LDS / spill filter");
  const size_t n = cand.size();
  auto launch = [&](const Candidate &c) { return launch_entry(*c.e, call, c.splits, workspace); };
  Events evs;
  int st = evs.create(n + 1);
  if (st != FA_OK) return st;
  auto &ev = evs.ev;
  // Warm up on the built-in default: one timed launch sizes the warm-up and the samples.
  if ((st = hip_status(hipEventRecord(ev[0], s), "hipEventRecord")) != FA_OK) return st;
  if ((st = launch(cand[first])) != FA_OK) return st;
  if ((st = hip_status(hipEventRecord(ev[1], s), "hipEventRecord")) != FA_OK) return st;
  if ((st = hip_status(hipEventSynchronize(ev[1]), "hipEventSynchronize")) != FA_OK) return st;
  float t1 = 0.f;
  if ((st = elapsed(ev[0], ev[1], &t1)) != FA_OK) return st;
  t1 = std::max(t1, 1e-3f);
  const int warm = (int)std::min(4000.f, std::ceil(kWarmMs / t1));
  const int reps = (int)std::min(256.f, std::max(1.f, std::ceil(kSampleMs / t1)));
  for (int i = 0; i < warm; ++i)
    if ((st = launch(cand[first])) != FA_OK) return st;
  for (const auto &c : cand)  // every candidate once, untimed (first-launch costs)
    if ((st = launch(c)) != FA_OK) return st;
  // Interleaved rounds: round r times candidate (i + r) % n in position i.
  std::vector<std::vector<float>> t(n);
  for (int r = 0; r < rounds; ++r) {
    if ((st = hip_status(hipEventRecord(ev[0], s), "hipEventRecord")) != FA_OK) return st;
    for (size_t i = 0; i < n; ++i) {
      for (int k = 0; k < reps; ++k)
        if ((st = launch(cand[(i + r) % n])) != FA_OK) return st;
      if ((st = hip_status(hipEventRecord(ev[i + 1], s), "hipEventRecord")) != FA_OK) return st;
    }
    if ((st = hip_status(hipEventSynchronize(ev[n]), "hipEventSynchronize")) != FA_OK) return st;
    for (size_t i = 0; i < n; ++i) {
      float ms = 0.f;
      if ((st = elapsed(ev[i], ev[i + 1], &ms)) != FA_OK) return st;
      t[(i + r) % n].push_back(ms / reps);
    }
  }
  for (size_t i = 0; i < n; ++i) cand[i].ms = median_of(t[i]);
  std::stable_sort(cand.begin(), cand.end(), [](const Candidate &a, const Candidate &b) { return a.ms < b.ms; });
  // The two best against each other, in alternating order, twice as many rounds.
  if (n >= 2) {
    std::vector<float> ta, tb;
    for (int r = 0; r < 2 * rounds; ++r) {
      const Candidate &x = r % 2 ? cand[1] : cand[0], &y = r % 2 ? cand[0] : cand[1];
      if ((st = hip_status(hipEventRecord(ev[0], s), "hipEventRecord")) != FA_OK) return st;
      for (int k = 0; k < reps; ++k)
        if ((st = launch(x)) != FA_OK) return st;
      if ((st = hip_status(hipEventRecord(ev[1], s), "hipEventRecord")) != FA_OK) return st;
      for (int k = 0; k < reps; ++k)
        if ((st = launch(y)) != FA_OK) return st;
      if ((st = hip_status(hipEventRecord(ev[2], s), "hipEventRecord")) != FA_OK) return st;
      if ((st = hip_status(hipEventSynchronize(ev[2]), "hipEventSynchronize")) != FA_OK) return st;
      float mx = 0.f, my = 0.f;
      if ((st = elapsed(ev[0], ev[1], &mx)) != FA_OK || (st = elapsed(ev[1], ev[2], &my)) != FA_OK) return st;
      (r % 2 ? tb : ta).push_back(mx / reps);
      (r % 2 ? ta : tb).push_back(my / reps);
    }
    cand[0].ms = median_of(ta);
    cand[1].ms = median_of(tb);
    if (cand[1].ms < cand[0].ms) std::swap(cand[0], cand[1]);
  }
  g_last_ranking.clear();
  for (const auto &c : cand) g_last_ranking.push_back(Ranked{cfg_of(*c.e), c.ms});
  *best = cand[0];
  return FA_OK;
}

}  // namespace

namespace fa {
int fwd_check_args(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
                   int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale, int causal,
                   const int32_t *cu_seqlens, int dtype) {
  return check_args(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale, causal,
                    cu_seqlens, dtype);
}
int set_error(int status, const char *msg) { return fail(status, msg); }
}  // namespace fa

extern "C" {

int fa_fwd_ext(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
               int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale, int causal,
               const int32_t *cu_seqlens, int dtype, int num_splits, void *workspace, size_t workspace_bytes,
               void *stream) {
  int st = check_args(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale, causal,
                      cu_seqlens, dtype);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS)
    return fail(FA_ERR_INVALID_ARG, "num_splits must be 0 (automatic) or 1 .. FA_MAX_SPLITS");
  const Shape shape{batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, dtype, cu_seqlens != nullptr,
                    causal != 0};
  const fa_tile_config_t c = choose_config(shape);
  if (num_splits == 0) num_splits = splits_within(c, shape, workspace, workspace_bytes);
  if (num_splits > 1) {
    if (!workspace) return fail(FA_ERR_INVALID_ARG, "num_splits > 1 needs a workspace");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(FA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    if (workspace_bytes < workspace_bytes_of(batch, seqlen_q, n_heads, d_head, num_splits))
      return fail(FA_ERR_INVALID_ARG, "workspace smaller than fa_fwd_workspace_bytes() for num_splits");
  }
  const KernelEntry *e = find_entry(dtype, d_head, c);
  if (!e) return fail(FA_ERR_UNSUPPORTED, "no compiled kernel for the chosen tile configuration");
  const Call call = make_call(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale,
                              causal, cu_seqlens, dtype, stream);
  return launch_entry(*e, call, num_splits, workspace);
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
           int seqlen_k, int n_heads, int d_head, float scale, const int32_t *cu_seqlens, int dtype,
           void *stream) {
  return fa_fwd_ext(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads, d_head, scale, 0, cu_seqlens,
                    dtype, 1, nullptr, 0, stream);
}

size_t fa_fwd_workspace_bytes(int batch, int seqlen_q, int n_heads, int d_head, int num_splits) {
  if (batch < 1 || seqlen_q < 1 || n_heads < 1 || num_splits < 1 || num_splits > FA_MAX_SPLITS) {
    fail(FA_ERR_INVALID_ARG, "batch, seqlen_q, n_heads must be >= 1 and num_splits in 1 .. FA_MAX_SPLITS");
    return 0;
  }
  if (!valid_d(d_head)) {
    fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
    return 0;
  }
  ok();
  return workspace_bytes_of(batch, seqlen_q, n_heads, d_head, num_splits);
}

int fa_fwd_choose_splits(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype, int causal,
                         int varlen) {
  if (!valid_dtype(dtype)) return fail(-FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (batch < 1 || n_heads < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(-FA_ERR_INVALID_ARG, "batch, n_heads, seqlen_q and seqlen_k must be >= 1");
  if (!valid_d(d_head)) return fail(-FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  ok();
  const Shape shape{batch, seqlen_q, seqlen_k, n_heads, n_heads, d_head, dtype, varlen != 0, causal != 0};
  return splits_for(choose_config(shape), shape);
}

size_t fa_bwd_workspace_bytes(int batch, int seqlen_q, int n_heads, int d_head, int atomic_dq) {
  if (batch < 1 || seqlen_q < 1 || n_heads < 1 || (atomic_dq != 0 && atomic_dq != 1)) {
    fail(FA_ERR_INVALID_ARG, "batch, seqlen_q and n_heads must be >= 1 and atomic_dq 0 or 1");
    return 0;
  }
  if (!valid_d(d_head)) {
    fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
    return 0;
  }
  ok();
  return bwd_bytes(batch, seqlen_q, n_heads, d_head, atomic_dq);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
           void *dq, void *dk, void *dv, int batch, int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv,
           int d_head, float scale, int causal, const int32_t *cu_seqlens, int dtype, int atomic_dq,
           void *workspace, size_t workspace_bytes, void *stream) {
  // dq stands in for the forward's o in the common checks; o, dout, dk, dv, workspace below
  int st = check_args(q, k, v, dq, const_cast<float *>(lse), batch, seqlen_q, seqlen_k, n_heads, n_heads_kv,
                      d_head, scale, causal, cu_seqlens, dtype);
  if (st != FA_OK) return st;
  if (!o || !dout || !dk || !dv) return fail(FA_ERR_INVALID_ARG, "o, dout, dk and dv must be non-null");
  if (atomic_dq != 0 && atomic_dq != 1) return fail(FA_ERR_INVALID_ARG, "atomic_dq must be 0 or 1");
  auto mis = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) % 16) != 0; };
  if (mis(o) || mis(dout) || mis(dk) || mis(dv))
    return fail(FA_ERR_MISALIGNED, "o, dout, dq, dk and dv must be 16-byte aligned");
  if (!workspace) return fail(FA_ERR_INVALID_ARG, "the backward pass needs a workspace");
  if (mis(workspace)) return fail(FA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (workspace_bytes < bwd_bytes(batch, seqlen_q, n_heads, d_head, atomic_dq))
    return fail(FA_ERR_INVALID_ARG, "workspace smaller than fa_bwd_workspace_bytes()");
  // the fp32 dQ rows of one sequence are addressed with 32-bit offsets (one query tile of slack)
  if (((int64_t)seqlen_q + 64) * n_heads * d_head * 4 >= (int64_t)INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "seqlen_q x n_heads x d_head too large for 32-bit offsets");
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu_seqlens = cu_seqlens;
  a.batch = batch;
  a.seqlen_q = seqlen_q;
  a.seqlen_k = seqlen_k;
  a.heads = n_heads;
  a.heads_kv = n_heads_kv;
  a.group = n_heads / n_heads_kv;
  a.causal = causal;
  const int bk = fa::bwd_block_keys(d_head);
  a.n_ktiles = (seqlen_k + bk - 1) / bk;
  a.total_wgs = batch * n_heads_kv * a.n_ktiles;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  float *ws = static_cast<float *>(workspace);
  const size_t rows = (size_t)batch * seqlen_q * n_heads;
  a.dq_acc = atomic_dq ? ws : nullptr;
  a.dvec = ws + (atomic_dq ? rows * d_head : 0);
  a.lse2 = a.dvec + rows;
  hipError_t err = fa::launch_bwd(a, d_head, dtype, reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("backward launch failed: ") + hipGetErrorString(err));
  return ok();
}

int fa_fwd_set_config(int d_head, int dtype, const fa_tile_config_t *cfg) {
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (!valid_d(d_head)) return fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  if (!cfg) {
    g_forced.erase({d_head, dtype});
    return ok();
  }
  if (!find_entry(dtype, d_head, *cfg))
    return fail(FA_ERR_UNSUPPORTED, "no compiled kernel for this tile configuration");
  g_forced[{d_head, dtype}] = *cfg;
  return ok();
}

int fa_fwd_get_config(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype,
                      int varlen, fa_tile_config_t *out) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "out must be non-null");
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (batch < 1 || n_heads < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(FA_ERR_INVALID_ARG, "batch, n_heads, seqlen_q and seqlen_k must be >= 1");
  if (!valid_d(d_head)) return fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  *out = choose_config(Shape{batch, seqlen_q, seqlen_k, n_heads, n_heads, d_head, dtype, varlen != 0, false});
  return ok();
}

int fa_fwd_get_config_ext(int batch, int seqlen_q, int seqlen_k, int n_heads, int d_head, int dtype,
                          int varlen, int causal, fa_tile_config_t *out) {
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  const int st = fa_fwd_get_config(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, varlen, out);
  if (st != FA_OK) return st;
  *out = choose_config(Shape{batch, seqlen_q, seqlen_k, n_heads, n_heads, d_head, dtype, varlen != 0, causal != 0});
  return ok();
}

int fa_fwd_query_config(int batch, int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, int dtype,
                        int varlen, int causal, fa_tile_config_t *out, int *num_splits, int *source) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "out must be non-null");
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (batch < 1 || n_heads < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(FA_ERR_INVALID_ARG, "batch, n_heads, seqlen_q and seqlen_k must be >= 1");
  if (n_heads_kv < 1 || n_heads % n_heads_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "n_heads_kv must be >= 1 and divide n_heads");
  if ((varlen != 0 && varlen != 1) || (causal != 0 && causal != 1))
    return fail(FA_ERR_INVALID_ARG, "varlen and causal must be 0 or 1");
  if (!valid_d(d_head)) return fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  const Shape shape{batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, dtype, varlen != 0, causal != 0};
  int src = kSrcDefault;
  *out = choose_config(shape, &src);
  if (num_splits) *num_splits = splits_for(*out, shape);
  if (source) *source = src;
  return ok();
}

int fa_fwd_num_configs(int d_head, int dtype) {
  if (!valid_dtype(dtype)) return fail(-FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (!valid_d(d_head)) return fail(-FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  int n = 0;
  for (const auto &e : entries()) n += (e.dtype == dtype && e.d_head == d_head);
  ok();
  return n;
}

int fa_fwd_list_configs(int d_head, int dtype, fa_tile_config_t *out, int capacity) {
  if (!valid_dtype(dtype)) return fail(-FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (!valid_d(d_head)) return fail(-FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  if (capacity < 0 || (capacity > 0 && !out)) return fail(-FA_ERR_INVALID_ARG, "bad output buffer");
  int n = 0;
  for (const auto &e : entries()) {
    if (e.dtype != dtype || e.d_head != d_head) continue;
    if (n < capacity) out[n] = cfg_of(e);
    ++n;
  }
  ok();
  return n;
}

int fa_fwd_config_lds_bytes(int d_head, const fa_tile_config_t *cfg) {
  if (!cfg) return fail(-FA_ERR_INVALID_ARG, "cfg must be non-null");
  if (!valid_d(d_head)) return fail(-FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  if (cfg->bc < 1 || cfg->stages < 1) return fail(-FA_ERR_INVALID_ARG, "bc and stages must be >= 1");
  ok();
  return lds_bytes_of(d_head, *cfg);
}

int fa_fwd_config_resources(int d_head, int dtype, const fa_tile_config_t *cfg, int *vgprs,
                            int *spill_bytes, int *lds_bytes) {
  if (!cfg) return fail(FA_ERR_INVALID_ARG, "cfg must be non-null");
  if (!valid_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "dtype must be FA_BF16 (0) or FA_FP16 (1)");
  if (!valid_d(d_head)) return fail(FA_ERR_UNSUPPORTED, "d_head must be 32, 64 or 128");
  const KernelEntry *e = find_entry(dtype, d_head, *cfg);
  if (!e) return fail(FA_ERR_UNSUPPORTED, "no compiled kernel for this tile configuration");
  hipFuncAttributes attr;
  hipError_t err = hipFuncGetAttributes(&attr, e->kernel);
  if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("hipFuncGetAttributes: ") + hipGetErrorString(err));
  if (vgprs) *vgprs = attr.numRegs;
  if (spill_bytes) *spill_bytes = (int)attr.localSizeBytes;
  if (lds_bytes) *lds_bytes = (int)attr.sharedSizeBytes;
  return ok();
}

int fa_fwd_autotune_ext(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int seqlen_q,
                        int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale, int causal,
                        const int32_t *cu_seqlens, int dtype, int num_splits, void *workspace,
                        size_t workspace_bytes, void *stream, int rounds, fa_tile_config_t *chosen,
                        float *best_ms) {
  int st = check_args(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale, causal,
                      cu_seqlens, dtype);
  if (st != FA_OK) return st;
  if (rounds < 1 || rounds > kMaxTuneRounds) return fail(FA_ERR_INVALID_ARG, "rounds must be 1 .. 100");
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS)
    return fail(FA_ERR_INVALID_ARG, "num_splits must be 0 (automatic) or 1 .. FA_MAX_SPLITS");
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(FA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (num_splits > 1 && (!workspace || workspace_bytes < workspace_bytes_of(batch, seqlen_q, n_heads, d_head,
                                                                             num_splits)))
    return fail(FA_ERR_INVALID_ARG, "num_splits > 1 needs a workspace of fa_fwd_workspace_bytes() bytes");
  const Shape shape{batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, dtype, cu_seqlens != nullptr,
                    causal != 0};
  const Call call = make_call(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale,
                              causal, cu_seqlens, dtype, stream);
  std::lock_guard<std::mutex> tlk(g_tune_mu);
  Candidate best;
  st = tune(call, shape, num_splits, workspace, workspace_bytes, rounds, &best);
  if (st != FA_OK) return st;
  bool saved = true;
  {
    std::lock_guard<std::mutex> lk(g_cfg_mu);
    g_tuned[key_of(shape)] = Tuned{cfg_of(*best.e), best.ms};
    if (const char *path = cache_path()) saved = save_cache_locked(path) == 0;
  }
  // Leave O and LSE holding the winner's result.
  st = launch_entry(*best.e, call, best.splits, workspace);
  if (st != FA_OK) return st;
  hipError_t err = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(err));
  if (chosen) *chosen = cfg_of(*best.e);
  if (best_ms) *best_ms = best.ms;
  if (!saved)
    return fail(FA_ERR_INVALID_ARG, std::string("tuned, but the cache file FA_FWD_TUNE_CACHE=") + cache_path() +
                                        " could not be written");
  return ok();
}

int fa_fwd_autotune(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                    int seqlen_q, int seqlen_k, int n_heads, int d_head, float scale,
                    const int32_t *cu_seqlens, int dtype, void *stream, int reps,
                    fa_tile_config_t *chosen, float *best_ms) {
  return fa_fwd_autotune_ext(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads, d_head, scale, 0,
                             cu_seqlens, dtype, 1, nullptr, 0, stream, reps, chosen, best_ms);
}

int fa_fwd_tune_ranking(fa_tile_config_t *cfgs, float *ms, int capacity) {
  if (capacity < 0 || (capacity > 0 && (!cfgs || !ms))) return fail(-FA_ERR_INVALID_ARG, "bad output buffers");
  std::lock_guard<std::mutex> tlk(g_tune_mu);
  const int n = (int)g_last_ranking.size();
  for (int i = 0; i < n && i < capacity; ++i) {
    cfgs[i] = g_last_ranking[i].cfg;
    ms[i] = g_last_ranking[i].ms;
  }
  ok();
  return n;
}

int fa_fwd_tune_reset(void) {
  std::lock_guard<std::mutex> tlk(g_tune_mu);
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  g_tuned.clear();
  g_last_ranking.clear();
  return ok();
}

int fa_fwd_tune_save(const char *path) {
  if (!path || !*path) return fail(FA_ERR_INVALID_ARG, "path must be a non-empty string");
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  if (save_cache_locked(path) != 0) return fail(FA_ERR_INVALID_ARG, std::string("cannot write ") + path);
  return ok();
}

int fa_fwd_tune_load(const char *path) {
  if (!path || !*path) return fail(-FA_ERR_INVALID_ARG, "path must be a non-empty string");
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  const int n = load_cache_locked(path);
  if (n < 0) return fail(-FA_ERR_INVALID_ARG, std::string("cannot read ") + path);
  ok();
  return n;
}

const char *fa_last_error(void) { return g_last_error.c_str(); }

const char *fa_version(void) { return "fa_fwd 0.2 (gfx950)"; }

}  // extern "C"
