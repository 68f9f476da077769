// Measurement helpers: the rates plain probe kernels reach on this GPU, the
// practical ceilings the hot kernels are compared with beside the nominal
// peaks.  The paged decode kernel is bound by HBM bandwidth ("PagedAttention"
// (robocikowo.com), Złożoność obliczeniowa); the chunked prefill, which
// computes the prompt's attention once per chunk ("PagedAttention et
// RadixAttention : parlons de KV Cache", the part on the two independent
// problems), by the matrix cores.
//
// Streaming read:
// Each workgroup reads one contiguous share of the buffer; each lane reads
// 16-byte chunks (a wave a contiguous 1 KiB run) with kUnroll independent
// loads in flight before any is used.  (Contiguous shares measured 3-5 %
// faster than workgroups striding over the whole buffer.)  The loads are
// non-temporal, as the decode kernel's K/V stream: a plain load also
// allocates each line in the Infinity Cache, and a 4 GiB stream read that
// way measured 6.2 TB/s against 7.0 TB/s.  The loaded words are folded by
// XOR into one word per workgroup, written to `sink`, so no load can be
// dropped.
//
// Tile read: the same loads over a list of fixed-size tiles at given indices
// (the decode kernel reads each (block, kv head) tile of K and V, 4 KiB at
// 70B shape, at scattered places of the pool).  Each wave reads whole tiles
// of a contiguous share of the list, 1 KiB per load instruction, two tiles
// in flight.  Indices are clamped to the pool, so every read stays inside it.
//
// Matrix-core rate: every wave issues v_mfma_f32_32x32x16_bf16 (the prefill
// kernel's product) into four independent accumulators, operands in
// registers, no memory traffic but one store per lane at the end.  Under
// such sustained matrix-core load the GPU lowers its clock below the
// nominal 2.4 GHz, so this rate is below the published dense peak.
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

constexpr int kTileUnroll = 2;

__global__ __launch_bounds__(kThreads) void tile_read_kernel(const char* __restrict__ base, int64_t tile_bytes,
                                                             const int32_t* __restrict__ ids, int64_t num_tiles,
                                                             int64_t max_tiles, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  const int64_t t0 = num_tiles * wave / nwaves, t1 = num_tiles * (wave + 1) / nwaves;
  const int64_t runs = tile_bytes / 1024;  // 1 KiB per wave-wide load
  auto tile_at = [&](int64_t t) {
    int64_t id = ids[t];
    id = id < 0 ? 0 : (id >= max_tiles ? max_tiles - 1 : id);
    return reinterpret_cast<const u32x4v*>(base + id * tile_bytes);
  };
  uint32_t acc = 0;
  int64_t t = t0;
  for (; t + kTileUnroll <= t1; t += kTileUnroll) {
    const u32x4v* tp[kTileUnroll];
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) tp[u] = tile_at(t + u);
    for (int64_t r = 0; r < runs; r += 4) {
      u32x4v v[kTileUnroll][4];
#pragma unroll
      for (int u = 0; u < kTileUnroll; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u][q] = r + q < runs ? __builtin_nontemporal_load(tp[u] + (r + q) * 64 + lane) : u32x4v{};
#pragma unroll
      for (int u = 0; u < kTileUnroll; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc ^= v[u][q].x ^ v[u][q].y ^ v[u][q].z ^ v[u][q].w;
    }
  }
  for (; t < t1; ++t) {
    const u32x4v* tp = tile_at(t);
    for (int64_t r = 0; r < runs; ++r) {
      const u32x4v v = __builtin_nontemporal_load(tp + r * 64 + lane);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t wv[kThreads / 64];
  if (lane == 0) wv[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kThreads / 64; ++w) x ^= wv[w];
    sink[blockIdx.x] = x;
  }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float float16v;
constexpr int kMfmaThreads = 512;  // 8 waves: 2 per SIMD
constexpr int kMfmaPerIter = 16;   // products per wave and iteration

__global__ __launch_bounds__(kMfmaThreads) void mfma_rate_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 15) * 0.0625f);
    b[i] = static_cast<__bf16>(static_cast<float>((lane ^ i) & 7) * 0.125f);
  }
  float16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaPerIter / 4; ++k) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
  sink[static_cast<int64_t>(blockIdx.x) * kMfmaThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int32_t pkv_tile_read(const void* base, size_t tile_bytes, size_t max_tiles, const int32_t* ids, int64_t num_tiles,
                      void* sink, int32_t sink_words, void* stream) {
  if (!base || !sink || (num_tiles > 0 && !ids)) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if ((reinterpret_cast<uintptr_t>(base) & 15u) != 0 || tile_bytes == 0 || tile_bytes % 1024 != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "base must be 16-byte aligned and tile_bytes a positive multiple of 1024");
  if (max_tiles == 0 || max_tiles > static_cast<size_t>(INT64_MAX) / tile_bytes)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_tiles %zu out of range", max_tiles);
  if (num_tiles < 0 || sink_words <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_tiles %lld < 0 or sink_words %d <= 0", static_cast<long long>(num_tiles),
                     sink_words);
  if (num_tiles == 0) return pkv::ok();
  const int64_t waves = (num_tiles + kTileUnroll - 1) / kTileUnroll;
  int64_t grid = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (grid > sink_words) grid = sink_words;
  tile_read_kernel<<<dim3(static_cast<uint32_t>(grid)), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(base), static_cast<int64_t>(tile_bytes), ids, num_tiles, static_cast<int64_t>(max_tiles),
      static_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "pkv_tile_read launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

int32_t pkv_mfma_rate(void* sink, int32_t workgroups, int32_t iters, void* stream) {
  if (!sink) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (workgroups <= 0 || iters < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "workgroups %d must be > 0 and iters %d >= 0", workgroups, iters);
  if (static_cast<int64_t>(workgroups) > static_cast<int64_t>(UINT32_MAX / kMfmaThreads))
    return pkv::fail(PKV_ERR_INVALID_ARG, "workgroups %d exceeds the %u a launch holds", workgroups,
                     static_cast<unsigned>(UINT32_MAX / kMfmaThreads));
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return pkv::fail(PKV_ERR_INVALID_ARG, "sink must be 4-byte aligned");
  mfma_rate_kernel<<<dim3(static_cast<uint32_t>(workgroups)), kMfmaThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<float*>(sink), iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "pkv_mfma_rate launch failed: %s", hipGetErrorString(e));
  return pkv::ok();
}

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
