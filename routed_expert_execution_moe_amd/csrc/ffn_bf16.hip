// Decode expert FFN kernels for one weight format (see ffn.h).
#include "ffn.h"

namespace moert {

hipError_t launch_ffn_bf16(moe_ctx* ctx, const void* x, int T, hipStream_t s) {
  return launch_ffn_typed<MOE_BF16>(ctx, x, T, s);
}

}  // namespace moert
