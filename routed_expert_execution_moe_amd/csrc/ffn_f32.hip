// Decode expert FFN kernels for one weight format (see ffn.h).
#include "ffn.h"

namespace moert {

hipError_t launch_ffn_f32(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  return launch_ffn_typed<MOE_F32>(ctx, x, T, s);
}

}  // namespace moert
