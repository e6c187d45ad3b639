// Matrix-core decode attention of libkvq (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {

bool mfma_decode_eligible(const kvq_kv_view&, int) { return false; }
int mfma_decode_parts(const kvq_kv_view&, int, int) { return 1; }
hipError_t launch_decode_mfma(const kvq_kv_view&, const void*, int, int, float, float*,
                              int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kvq
