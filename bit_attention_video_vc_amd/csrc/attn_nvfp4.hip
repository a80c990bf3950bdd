// 4-bit V-Smooth path (NVFP4 residual, fp32 softmax, bf16 P.V): not built yet.
#include "attn_common.h"

int vc_attn_nvfp4_launch(const uint8_t*, const float*, const uint8_t*, const float*, const uint8_t*,
                         const float*, const uint8_t*, const uint16_t*, int, int, int, float, float*,
                         hipStream_t) {
  return VC_ERR_UNSUPPORTED;
}
