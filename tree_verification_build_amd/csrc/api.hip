// Host-side plumbing shared by every entry point: status messages, the
// sampling constants and the version string.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "common.hpp"

namespace ddt {

static thread_local char g_err[512] = "";

ddtree_status fail(ddtree_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ddtree_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DDTREE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return DDTREE_OK;
}

// c = fp32(log2(e) / T) with T as given in fp32 and log2(e) the nearest double;
// a[n] = fp32((ln 2)^n / n!) evaluated in long double, then rounded once.
WeightConsts weight_consts(float temperature) {
  WeightConsts w;
  w.c = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  long double ln2 = 0.693147180559945309417232121458176568L;
  long double term = 1.0L;
  for (int n = 0; n < 7; ++n) {
    w.a[n] = static_cast<float>(term);
    term = term * ln2 / static_cast<long double>(n + 1);
  }
  return w;
}

}  // namespace ddt

extern "C" {

const char* ddtree_last_error(void) { return ddt::g_err; }

const char* ddtree_version(void) { return "libddtree 0.1 gfx950"; }

ddtree_status ddtree_sampling_constants(float temperature, float* c, float* a7) {
  if (!(temperature > 0.0f) || !std::isfinite(temperature))
    return ddt::fail(DDTREE_EINVAL, "sampling_constants: temperature must be > 0 and finite");
  if (!c || !a7) return ddt::fail(DDTREE_EINVAL, "sampling_constants: null output pointer");
  ddt::WeightConsts w = ddt::weight_consts(temperature);
  *c = w.c;
  for (int n = 0; n < 7; ++n) a7[n] = w.a[n];
  return DDTREE_OK;
}

}  // extern "C"
