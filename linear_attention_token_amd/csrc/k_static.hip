// Allocation-free prefill: gdn_prefill with the workspace taken from a static device array.
//
// The array lives in the library's code object, so every GPU the library runs on holds its own copy
// at its own address. In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device with that device current, and only
// that address is ever handed to a kernel.
#include <mutex>

#include "gdn_internal.h"

static __device__ __align__(256) unsigned char scratch[GDN_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch`, looked up on the first call there. (The
// caller's stream must belong to that device, as for every HIP launch.)
gdn_status device_scratch(hipStream_t, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gdn::report(GDN_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return gdn::report(GDN_E_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gdn::report(GDN_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_prefill_static(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                                         const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                         const void* q, const void* k, const void* v,
                                         int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                         const float* alpha, const float* beta, const void* gate,
                                         const float* conv_w, const float* norm_w,
                                         const float* state_in, float* state_out,
                                         const void* conv_in, void* conv_out, void* out, void* hip_stream) {
  return gdn::prefill_with(cfg, n_seqs, total_tokens, cu_seqlens, cu_seqlens_host, q, k, v, ld_q, ld_k, ld_v,
                           alpha, beta, gate, conv_w, norm_w, state_in, state_out, conv_in, conv_out, out, nullptr,
                           GDN_STATIC_WORKSPACE_BYTES, device_scratch, hip_stream);
}
