// Library-wide entry points of libspectree: ABI version and the per-thread error string.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "api_common.h"

namespace spectree {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

}  // namespace spectree

extern "C" int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

extern "C" const char* spec_last_error(void) { return spectree::g_last_error.c_str(); }
