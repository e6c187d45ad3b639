// Decode attention for callers that cannot allocate device memory: the
// split partials live in a fixed array of the library's own device memory
// instead of a caller workspace.
#include <hip/hip_runtime.h>
#include <mutex>

#include "kvq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)KVQ_NOALLOC_SCRATCH_BYTES;

// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// only the address from hipGetSymbolAddress below is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device

// The array's device address on the current device (looked up once per
// device, with that device current), or null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention_noalloc(const kvq_kv_view* v, const void* q, int dtype,
                                        int n_q_heads, float sm_scale, float* out,
                                        int n_splits, int flags, void* stream) {
  const size_t need = kvq_decode_workspace_bytes(v, n_q_heads, n_splits);
  if (need == 0) return KVQ_E_ARG;
  if (need > kScratchBytes) return KVQ_E_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return KVQ_E_HIP;
  return kvq::decode_attention_impl(v, q, dtype, n_q_heads, sm_scale, out, n_splits, flags, ws,
                                    kScratchBytes, stream);
}

}  // extern "C"
