// fa_fwd_noalloc.hip -- fa_fwd_ext for callers that cannot allocate device memory: code
// under stream capture, tight serving loops, harnesses that forbid hipMalloc.
//
// fa_fwd_ext's only scratch memory is the split path's: each split's fp32 partial output
// rows and natural-log LSE rows, which the merge kernel reads back.  fa_fwd_ext takes it
// from a caller workspace; fa_fwd_ext_noalloc takes it from `scratch`, a file-scope device
// array of FA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
// process ends.  Nothing here calls hipMalloc, hipFree or any allocating routine.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address
// is obtained once per device, with that device current, by hipGetSymbolAddress, and only
// that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's contents.
// Nothing in it needs to start at zero: every split workgroup writes all rows of its own
// partial slab (zeros and -inf for a share with no visible key) before the merge reads
// them.  Calls that overlap in time on one GPU (different streams, or threads racing on one
// stream) race on the array; order them on one stream.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>

#include "fa_fwd.h"
#include "fa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
std::map<int, void *> g_scratch_of;  // device ordinal -> device address of its `scratch`

// Device address of the current device's `scratch`, resolved on the first call per device.
int scratch_on_current_device(void **ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return fa::set_error(FA_ERR_HIP, (std::string("hipGetDevice: ") + hipGetErrorString(err)).c_str());
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch_of.find(dev);
  if (it != g_scratch_of.end()) {
    *ptr = it->second;
    return FA_OK;
  }
  void *p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess || !p)
    return fa::set_error(FA_ERR_HIP, (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(err)).c_str());
  g_scratch_of[dev] = p;
  *ptr = p;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_ext_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                  int seqlen_q, int seqlen_k, int n_heads, int n_heads_kv, int d_head, float scale,
                                  int causal, const int32_t *cu_seqlens, int dtype, int num_splits, void *stream) {
  int st = fa::fwd_check_args(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale,
                              causal, cu_seqlens, dtype);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS)
    return fa::set_error(FA_ERR_INVALID_ARG, "num_splits must be 0 (automatic) or 1 .. FA_MAX_SPLITS");
  if (num_splits > 1) {
    const size_t need = fa_fwd_workspace_bytes(batch, seqlen_q, n_heads, d_head, num_splits);
    if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) {
      const std::string msg = "num_splits = " + std::to_string(num_splits) + " needs " + std::to_string(need) +
                              " bytes of scratch; fa_fwd_ext_noalloc holds FA_NOALLOC_SCRATCH_BYTES = " +
                              std::to_string((size_t)FA_NOALLOC_SCRATCH_BYTES) +
                              " (use fewer splits, 0 for automatic, or fa_fwd_ext with a workspace)";
      return fa::set_error(FA_ERR_INVALID_ARG, msg.c_str());
    }
  }
  void *ws = nullptr;
  if (num_splits != 1) {
    st = scratch_on_current_device(&ws);
    if (st != FA_OK) return st;
  }
  // num_splits = 0: fa_fwd_ext lowers the automatic count to what the scratch holds
  return fa_fwd_ext(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head, scale, causal,
                    cu_seqlens, dtype, num_splits, ws, ws ? (size_t)FA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
