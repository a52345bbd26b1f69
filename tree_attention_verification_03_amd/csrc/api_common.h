// Host-side helpers shared by the extern "C" entry points of libspectree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/spec_tree.h"

namespace spectree {

// Thread-local message of the last failing call (defined in api.cpp).
void set_error(const char* fmt, ...);
void clear_error();

inline int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  set_error("%s", buf);
  return code;
}

inline int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SPEC_E_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  clear_error();
  return SPEC_OK;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
inline int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace spectree
