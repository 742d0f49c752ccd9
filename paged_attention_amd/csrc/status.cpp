// Status strings and the per-thread last-error detail.
#include "status.h"

#include <cstdio>

namespace pkv {

namespace {
thread_local char g_last_error[512] = "";
thread_local CallEvents g_call_events;
}

void set_call_events(const CallEvents& e) { g_call_events = e; }

CallEvents take_call_events() {
  const CallEvents e = g_call_events;
  g_call_events = CallEvents{};
  return e;
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

const char* last_error() { return g_last_error; }

}  // namespace pkv

extern "C" {

PKV_API const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_NO_BLOCKS: return "out of blocks";
    case PKV_ERR_BAD_BLOCK: return "block id out of range";
    case PKV_ERR_REFCOUNT: return "reference count error";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

PKV_API const char* pkv_last_error(void) { return pkv::last_error(); }

PKV_API int pkv_version(void) { return 100; }

PKV_API int pkv_time_next_decode(hipEvent_t start, hipEvent_t stop) {
  pkv::set_call_events(pkv::CallEvents{start, stop});
  return PKV_OK;
}

}  // extern "C"
