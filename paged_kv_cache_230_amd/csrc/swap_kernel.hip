// Swap copies for the paged KV cache on gfx950: whole blocks between the
// device pool and a host swap pool of the same format, either way
// ("PagedAttention — Gestion mémoire pour LLM à long contexte", Mode d'échec
// and the glossary's Page eviction: when GPU memory runs out even with
// paging, pages go to CPU RAM and are read back on demand).  A pinned host
// pool is read or written in place over the bus through its device mapping;
// pageable host memory is rejected.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_status.h"

namespace {

int32_t check_common(int32_t head_dim, int32_t block_size, pkv_dtype dt) {
  if (dt != PKV_F32 && dt != PKV_BF16) return pkv::fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
  if (head_dim != 64 && head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported (16 or 32)", block_size);
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return pkv::ok();
}

// Swap copy between two pools of the same format, either of which may be
// pinned host memory read or written in place over the bus: blockIdx.x =
// pair, blockIdx.y = 0 (K) or 1 (V).  Pairs naming blocks outside either
// pool are skipped and set the bad-pair flag of the device status word.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const char* __restrict__ src_k,
                                                          const char* __restrict__ src_v, char* __restrict__ dst_k,
                                                          char* __restrict__ dst_v, const int32_t* __restrict__ pairs,
                                                          int64_t block_bytes, int32_t src_blocks,
                                                          int32_t dst_blocks, int32_t* __restrict__ status) {
  const int pair = blockIdx.x;
  const int32_t s = pairs[2 * pair];
  const int32_t d = pairs[2 * pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) {
    if (threadIdx.x == 0 && blockIdx.y == 0)
      __hip_atomic_fetch_or(status, PKV_DEV_BAD_PAIR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const char* from = (blockIdx.y == 0 ? src_k : src_v) + static_cast<int64_t>(s) * block_bytes;
  char* to = (blockIdx.y == 0 ? dst_k : dst_v) + static_cast<int64_t>(d) * block_bytes;
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
    reinterpret_cast<uint4*>(to)[i] = reinterpret_cast<const uint4*>(from)[i];
}

// Address a kernel can use for `p`: device memory as is, pinned host memory
// through its device mapping; anything else (pageable host memory) is an
// error.
int32_t kernel_address(const void* p, const char* name, const char** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return pkv::fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", name);
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return pkv::fail(PKV_ERR_INVALID_ARG, "%s is host memory without a device mapping", name);
    }
    *out = static_cast<const char*>(d);
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = static_cast<const char*>(p);
    return PKV_OK;
  }
  return pkv::fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", name);
}

}  // namespace

extern "C" int32_t paged_kv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                        const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t src_num_blocks,
                                        int32_t dst_num_blocks, pkv_dtype dt, void* stream) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (num_pairs < 0 || num_kv_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes: num_pairs %d num_kv_heads %d src_num_blocks %d dst_num_blocks %d",
                     num_pairs, num_kv_heads, src_num_blocks, dst_num_blocks);
  if (num_pairs == 0) return pkv::ok();
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const char *sk, *sv, *dk, *dv, *pr;
  if (int32_t e = kernel_address(src_k, "src_k", &sk)) return e;
  if (int32_t e = kernel_address(src_v, "src_v", &sv)) return e;
  if (int32_t e = kernel_address(dst_k, "dst_k", &dk)) return e;
  if (int32_t e = kernel_address(dst_v, "dst_v", &dv)) return e;
  if (int32_t e = kernel_address(pairs, "pairs", &pr)) return e;
  const int eb = dt == PKV_BF16 ? 2 : 4;
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * eb;
  int32_t* status = nullptr;
  if (int32_t e = pkv::device_status_ptr(&status)) return e;
  swap_blocks_kernel<<<dim3(num_pairs, 2), 256, 0, static_cast<hipStream_t>(stream)>>>(
      sk, sv, const_cast<char*>(dk), const_cast<char*>(dv), reinterpret_cast<const int32_t*>(pr), block_bytes,
      src_num_blocks, dst_num_blocks, status);
  return launch_status("paged_kv_swap_blocks");
}
