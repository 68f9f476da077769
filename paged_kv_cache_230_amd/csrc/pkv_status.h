// Internal: per-thread error reporting shared by the library's sources.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/pagedkv.h"

namespace pkv {

std::string& last_error_slot();

// Records a printf-style message for pkv_last_error() and returns `code`.
inline int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return code;
}

inline int32_t ok() {
  last_error_slot().clear();
  return PKV_OK;
}

}  // namespace pkv
