// Status strings and the thread-local record of the last HIP launch error.
#include <hip/hip_runtime.h>

#include "../../include/vc.h"

static thread_local int g_last_hip_error = 0;

int vc_set_hip_error(int hip_error) {
  g_last_hip_error = hip_error;
  return VC_ERR_HIP;
}

extern "C" int vc_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char* vc_status_string(int status) {
  switch (status) {
    case VC_OK: return "ok";
    case VC_ERR_INVALID_ARG: return "invalid argument";
    case VC_ERR_UNSUPPORTED: return "unsupported shape or mode";
    case VC_ERR_WORKSPACE: return "workspace missing or too small";
    case VC_ERR_HIP: return hipGetErrorString(static_cast<hipError_t>(g_last_hip_error));
    default: return "unknown status";
  }
}

extern "C" const char* vc_version(void) { return "vc-attn-mi355x 0.1 (gfx950)"; }
