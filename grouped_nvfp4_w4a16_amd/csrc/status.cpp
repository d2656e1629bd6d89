// Status strings and the per-thread error message of the C ABI.
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace moe {

static thread_local char g_last_error[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace moe

extern "C" const char *moe_w4a16_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ECAPACITY: return "output buffer too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" const char *moe_w4a16_last_error(void) { return moe::g_last_error; }

#ifndef MOE_W4A16_SOURCE_SHA256
#define MOE_W4A16_SOURCE_SHA256 "unknown"
#endif

// The tag lets a reader find the hash in the file without loading the library.
static const char g_source_tag[] = "moe_w4a16_source_sha256=" MOE_W4A16_SOURCE_SHA256;

extern "C" const char *moe_w4a16_source_sha256(void) {
  return g_source_tag + sizeof("moe_w4a16_source_sha256=") - 1;
}
