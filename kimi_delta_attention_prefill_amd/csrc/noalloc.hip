// kda_prefill_noalloc: kda_prefill for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The split route's workspace (chunk records and window
// states) comes from a file-scope device array instead of the caller.
//
// The array is a symbol of this library's code object, so every GPU the
// library runs on holds its own copy (kNoallocScratchBytes) from the first
// call on that device until the process ends.  In host code its name is only
// a host-side stand-in; the device address is resolved once per device with
// hipGetSymbolAddress and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kNoallocScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of `scratch` on device `dev` (current), resolved once.
hipError_t scratch_address(int dev, void** out) {
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t num_heads, int32_t head_dim_k,
                                   int32_t head_dim_v, float scale, float lower_bound,
                                   const float* initial_state, float* final_state, void* out,
                                   hipStream_t stream) {
  // Sizes first: kda_prefill_workspace_size is a host function of the sizes
  // and the route the planner picks (0 for invalid sizes, which kda_prefill
  // then reports).
  const size_t need = kda_prefill_workspace_size(num_seqs, total_tokens, num_heads);
  if (need > kNoallocScratchBytes)
    return kda::set_error(KDA_ERR_WORKSPACE,
                          "kda_prefill_noalloc: this problem needs %zu bytes of workspace, more "
                          "than the %zu-byte static scratch (use kda_prefill with a workspace)",
                          need, kNoallocScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return kda::set_error(KDA_ERR_HIP, "kda_prefill_noalloc: hipGetDevice failed: %s",
                          hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return kda::set_error(KDA_ERR_UNSUPPORTED, "kda_prefill_noalloc: device %d out of range", dev);
  void* ws = nullptr;
  if ((e = scratch_address(dev, &ws)) != hipSuccess || !ws)
    return kda::set_error(KDA_ERR_HIP,
                          "kda_prefill_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                          hipGetErrorString(e));
  return kda_prefill(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim_k,
                     head_dim_v, scale, lower_bound, initial_state, final_state, out, ws,
                     kNoallocScratchBytes, stream);
}
