// Status strings and the thread-local record of the last HIP launch error.
#include <hip/hip_runtime.h>

#include <cmath>

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
    case VC_ERR_SCRATCH: return "problem too large for the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

// Grouping cadence (see vc.h): steps s < fraction * total_steps form the window,
// in which every reuse-th step regroups.
static int group_window(int total_steps, int reuse, float fraction) {
  if (total_steps < 1 || reuse < 1 || !(fraction > 0.0f) || fraction > 1.0f) return VC_ERR_INVALID_ARG;
  const double x = (double)fraction * (double)total_steps;   // window = integers s with s < x
  int w = (int)std::ceil(x);
  if (w < 1) w = 1;
  if (w > total_steps) w = total_steps;
  return w;
}

extern "C" int vc_group_due(int step, int total_steps, int reuse, float fraction) {
  const int w = group_window(total_steps, reuse, fraction);
  if (w < 0) return w;
  if (step < 0 || step >= total_steps) return VC_ERR_INVALID_ARG;
  return (step < w && step % reuse == 0) ? 1 : 0;
}

extern "C" int vc_group_source(int step, int total_steps, int reuse, float fraction) {
  const int w = group_window(total_steps, reuse, fraction);
  if (w < 0) return w;
  if (step < 0 || step >= total_steps) return VC_ERR_INVALID_ARG;
  const int last = step < w ? step : w - 1;   // latest window step at or before `step`
  return last - last % reuse;
}

extern "C" int vc_group_count(int total_steps, int reuse, float fraction) {
  const int w = group_window(total_steps, reuse, fraction);
  if (w < 0) return w;
  return (w - 1) / reuse + 1;
}

extern "C" const char* vc_version(void) { return "vc-attn-mi355x 0.1 (gfx950)"; }
