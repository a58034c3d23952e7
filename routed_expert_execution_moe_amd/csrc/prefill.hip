// Prefill compute: grouped expert GEMM over a full-layer buffer (in progress).
#include "internal.h"

namespace moert {

hipError_t launch_prefill_compute(moe_ctx*, int, const void*, int, const int32_t*, const float*,
                                  void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moert
