#include "ta_error.h"

namespace {
thread_local char g_err[512] = "";
}

namespace ta {

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace ta

extern "C" const char* tree_attn_last_error(void) { return g_err; }
