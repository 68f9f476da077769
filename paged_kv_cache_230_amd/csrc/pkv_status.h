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

// Device address of a pinned host buffer (error if it is not pinned).
int32_t stage_device_ptr(const int32_t* stage, const int32_t** dev);

// Device address of the current GPU's status word (kernels OR PKV_DEV_*
// flags into it); an error status if the device or the symbol is unusable.
int32_t device_status_ptr(int32_t** out);

// Launches the staging kernel that copies one decode step's record from
// pinned host memory (read in place by the GPU, at `stage_dev`) into the
// device buffers.
int32_t launch_stage(const int32_t* stage_dev, int32_t n_seqs, int32_t n_pairs, int32_t n_updates, int32_t width,
                     int32_t* slot_mapping, int32_t* context_lens, int32_t* cow_pairs, int32_t* block_tables,
                     void* stream);

inline int32_t ok() {
  last_error_slot().clear();
  return PKV_OK;
}

}  // namespace pkv
