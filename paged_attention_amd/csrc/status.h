// Status codes and the per-thread error detail shared by every libpkv source.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Rows, pools and queries are moved 16 bytes per lane: their base addresses
// must be 16-byte aligned (null counts as aligned; callers check it apart).
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Records a formatted detail for pkv_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_error();

// The calling thread's pending kernel-timing request for its next decode call
// (pkv_time_next_decode); taking it clears it.
struct CallEvents {
  hipEvent_t start = nullptr;  // recorded at the start of the call's first kernel
  hipEvent_t stop = nullptr;   // recorded at the end of its last kernel
};
void set_call_events(const CallEvents& e);
CallEvents take_call_events();

}  // namespace pkv
