// Measurement helper: the HBM read rate a plain streaming kernel reaches on
// this GPU, the practical ceiling a bandwidth-bound kernel is compared with
// beside the nominal peak.  The paged decode kernel is bound by HBM
// bandwidth ("PagedAttention" (robocikowo.com), Złożoność obliczeniowa), so
// its achieved rate is reported against both.
//
// Each workgroup reads one contiguous share of the buffer; each lane reads
// 16-byte chunks (a wave a contiguous 1 KiB run) with kUnroll independent
// loads in flight before any is used.  (Contiguous shares measured 3-5 %
// faster than workgroups striding over the whole buffer.)  The loads are
// non-temporal, as the decode kernel's K/V stream: a plain load also
// allocates each line in the Infinity Cache, and a 4 GiB stream read that
// way measured 6.2 TB/s against 7.0 TB/s.  The loaded words are folded by
// XOR into one word per workgroup, written to `sink`, so no load can be
// dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_status.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n,
                                                               uint32_t* __restrict__ sink) {
  const int64_t c0 = n * blockIdx.x / gridDim.x, c1 = n * (blockIdx.x + 1) / gridDim.x;
  int64_t i = c0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < c1; i += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(buf + i + u * kThreads)));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < c1; i += kThreads) {
    const uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(buf + i)));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the workgroup's words into one
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t wv[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wv[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kThreads / 64; ++w) x ^= wv[w];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" {

int32_t pkv_stream_read(const void* buf, size_t bytes, void* sink, int32_t sink_words, void* stream) {
  if (!buf || !sink) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes % 16 != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "buffer must be 16-byte aligned and a multiple of 16 bytes");
  if (sink_words <= 0) return pkv::fail(PKV_ERR_INVALID_ARG, "sink_words %d <= 0", sink_words);
  if (bytes == 0) return pkv::ok();
  const int64_t n = static_cast<int64_t>(bytes / 16);
  int64_t grid = (n + kThreads - 1) / kThreads;
  if (grid > sink_words) grid = sink_words;
  stream_read_kernel<<<dim3(static_cast<uint32_t>(grid)), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), n, static_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "pkv_stream_read launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

}  // extern "C"
