// fa_quant_attention_static_ws: attention for callers that cannot allocate
// device memory.  The kernels' workspace (K / V re-layout images, per-tile
// scale data, key-split partial results) lives in one static device array
// per GPU instead of a caller-supplied buffer.  Nothing in that workspace
// has to start at zero: every byte a call reads was written earlier in the
// same call (k_prep fills every tile it covers, padding rows included, and
// each key split writes the partial rows k_combine reads), so the contents
// a previous call left behind are never read.

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = FA_QUANT_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

// The workspace of every call on a GPU.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address comes from
// hipGetSymbolAddress, once per device (with that device current), and
// only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];

// Device address of the current device's array (looked up on the first
// call on that device), or NULL with the HIP error in *err.
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" faq_status fa_quant_attention_static_ws(const faq_qtensor* q, const faq_qtensor* k,
                                                   const faq_qtensor* v, float sm_scale, int32_t causal, void* out,
                                                   int32_t out_dtype, void* stream) {
  static const char* fn = "fa_quant_attention_static_ws";
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (!ws) return FAQ_ERR_HIP;
  // validation, then the workspace check against the array's size: a call
  // that needs more returns FAQ_ERR_WORKSPACE and enqueues nothing
  return faq::attention_entry(q, k, v, sm_scale, causal, out, out_dtype, ws, kScratchBytes, stream, fn);
}
