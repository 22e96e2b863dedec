#include "status.h"

namespace orca {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

}  // namespace orca

extern "C" const char* orca_status_str(orca_status s) {
  switch (s) {
    case ORCA_OK: return "ORCA_OK";
    case ORCA_ERR_INVALID: return "ORCA_ERR_INVALID";
    case ORCA_ERR_NOSPACE: return "ORCA_ERR_NOSPACE";
    case ORCA_ERR_HIP: return "ORCA_ERR_HIP";
    case ORCA_ERR_UNSUPPORTED: return "ORCA_ERR_UNSUPPORTED";
  }
  return "ORCA_ERR_UNKNOWN";
}

extern "C" const char* orca_last_error(void) { return orca::g_last_error.c_str(); }
