// Status codes and the per-thread error detail shared by every libpkv source.
#pragma once

#include <cstdarg>

#include "pkv.h"

namespace pkv {

// Records a formatted detail for pkv_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_error();

}  // namespace pkv
