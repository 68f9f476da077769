// Paged KV-cache kernels for gfx950 (MI355X): cache append, copy-on-write
// block copy, split-context decode attention and the log-sum-exp merge.
//
// Method sources (page title, section):
//   "PagedAttention" (robocikowo.com), Jak działa / Komponenty: the attention
//     kernel reads a non-contiguous cache through the per-sequence block
//     table; the bottleneck is HBM bandwidth (Złożoność obliczeniowa).
//   "PagedAttention et RadixAttention : parlons de KV Cache" (aitalk.it),
//     PagedAttention section: blocks of 16 or 32 tokens (step 1), the table
//     consulted to collect the blocks (step 2), growth one block at a time
//     (step 3), shared blocks copied only on divergence (step 4), and the
//     attention result unchanged by paging (closing paragraph).
//
// Decode kernel design (gfx950, wave64):
//   * One workgroup = 4 waves = one (context partition, kv head, sequence).
//     Wave w walks the partition's blocks w, w+4, ...; each block tile of
//     one kv head is contiguous, and the pool layout makes every K and V
//     operand load a whole-wavefront contiguous run.
//   * QK^T runs on the matrix cores: 16 tokens x 16 query-head columns per
//     MFMA tile, with the G query heads that share the kv head in the
//     columns, so each K byte fetched serves all G heads.  The fp32 score
//     tile comes out in the exact lane layout the PV MFMA wants for P.
//   * Online softmax in the log2 domain (scale * log2(e) folded into the
//     fp32 scores), block max by cross-lane shuffles, rescale of the
//     accumulators only when a running max grows.
//   * PV on the matrix cores.  For bf16, P is split into a bf16 high part
//     (rows 0..7 of the A tile) and the bf16 rounding of the remainder (rows
//     8..15, the padding rows a group of <= 8 heads leaves free), so P is
//     carried to ~2^-17 relative precision at no extra MFMA cost; the two
//     halves are summed at the end.  fp32 uses the fp32 MFMA directly.
//   * The 4 waves merge in LDS; a sequence that fits one partition writes
//     the output, otherwise the partition writes (max, sum, unnormalised
//     accumulator) partials and a merge kernel combines them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pkv_status.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(4))) float float4v;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Lane value from lane (row + 8) mod 16 of the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float row_rotate8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;  // [S][Hq][max_parts][D]
  float* ws_m;    // [S][Hq][max_parts]
  float* ws_l;    // [S][Hq][max_parts]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t partition_size;
  int32_t max_parts;
  float scale_log2;  // scale * log2(e)
};

// ---------------------------------------------------------------------------
// Operand staging for one 16-token step of one (block, kv head) tile.
// bf16: K operand = D/32 x 16 B (8 dims of token `row`), V operand = D/16 x
// 8 B (4 tokens of dim 16*nt + row).  fp32: K = D/16 x 16 B (4 dims), V =
// D/16 x 16 B (4 tokens).
template <bool BF16, int D>
struct Step;

template <int D>
struct Step<true, D> {
  static constexpr int KK = D / 32;
  static constexpr int NT = D / 16;
  uint4 k[KK];
  uint2 v[NT];
};

template <int D>
struct Step<false, D> {
  static constexpr int KK = D / 16;
  static constexpr int NT = D / 16;
  float4 k[KK];
  float4 v[NT];
};

// Issue the loads of half `h` (16 tokens) of a block tile.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void load_step(Step<BF16, D>& st, const void* k_tile, const void* v_tile, int h, int row,
                                          int quad) {
  if constexpr (BF16) {
    const uint16_t* kt = static_cast<const uint16_t*>(k_tile);
    const uint16_t* vt = static_cast<const uint16_t*>(v_tile);
#pragma unroll
    for (int kk = 0; kk < Step<BF16, D>::KK; ++kk)
      st.k[kk] = *reinterpret_cast<const uint4*>(kt + ((4 * kk + quad) * BS + 16 * h + row) * 8);
#pragma unroll
    for (int nt = 0; nt < Step<BF16, D>::NT; ++nt)
      st.v[nt] = *reinterpret_cast<const uint2*>(vt + (16 * nt + row) * BS + 16 * h + 4 * quad);
  } else {
    const float* kt = static_cast<const float*>(k_tile);
    const float* vt = static_cast<const float*>(v_tile);
#pragma unroll
    for (int kk = 0; kk < Step<BF16, D>::KK; ++kk)
      st.k[kk] = *reinterpret_cast<const float4*>(kt + ((4 * kk + quad) * BS + 16 * h + row) * 4);
#pragma unroll
    for (int nt = 0; nt < Step<BF16, D>::NT; ++nt)
      st.v[nt] = *reinterpret_cast<const float4*>(vt + (16 * nt + row) * BS + 16 * h + 4 * quad);
  }
}

// Zero the V entries of tokens at or past `end` (their slots may hold
// anything, including NaN, and 0 * NaN would poison the accumulator).
template <bool BF16, int D>
__device__ __forceinline__ void mask_v(Step<BF16, D>& st, int tok0, int end) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool valid = tok0 + i < end;
#pragma unroll
    for (int nt = 0; nt < Step<BF16, D>::NT; ++nt) {
      if constexpr (BF16) {
        uint32_t& w = (i < 2) ? st.v[nt].x : st.v[nt].y;
        const uint32_t keep = (i & 1) ? 0xFFFF0000u : 0x0000FFFFu;
        if (!valid) w &= ~keep;
      } else {
        float& f = (i == 0) ? st.v[nt].x : (i == 1) ? st.v[nt].y : (i == 2) ? st.v[nt].z : st.v[nt].w;
        if (!valid) f = 0.f;
      }
    }
  }
}

template <bool BF16, int D>
struct QOperand;

template <int D>
struct QOperand<true, D> {
  bf16x8 q[D / 32];
};

template <int D>
struct QOperand<false, D> {
  float4 q[D / 16];
};

// Per-wave running state for one 16-row accumulator tile set.
template <int D>
struct Acc {
  float4v o[D / 16];
};

template <bool BF16, int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeArgs a) {
  constexpr int GMAX = BF16 ? 8 : 16;
  constexpr int NT = D / 16;
  __shared__ float sm_o[kWaves][GMAX][D];
  __shared__ float sm_m[kWaves][GMAX];
  __shared__ float sm_l[kWaves][GMAX];

  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int quad = lane >> 4;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int P = a.partition_size;

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  const size_t out_row0 = (static_cast<size_t>(s) * Hq + static_cast<size_t>(g) * G) * D;

  if (L == 0) {
    if (p == 0) {
      for (int e = threadIdx.x; e < G * D; e += kThreads) {
        if constexpr (BF16)
          static_cast<uint16_t*>(a.out)[out_row0 + e] = 0;
        else
          static_cast<float*>(a.out)[out_row0 + e] = 0.f;
      }
    }
    return;
  }
  const int start = p * P;
  if (start >= L) return;
  const int end = min(start + P, L);
  const int nparts = (L + P - 1) / P;
  const int nblk = (end - start + BS - 1) / BS;
  const int32_t* tbl = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq + start / BS;

  // Query operand: column `row` = query head g*G + row (zero past G).
  QOperand<BF16, D> qo;
  {
    const bool live = row < G;
    const size_t qoff = out_row0 + static_cast<size_t>(live ? row : 0) * D;
    if constexpr (BF16) {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qoff;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        uint4 u = live ? *reinterpret_cast<const uint4*>(qp + 32 * kk + 8 * quad) : make_uint4(0, 0, 0, 0);
        qo.q[kk] = __builtin_bit_cast(bf16x8, u);
      }
    } else {
      const float* qp = static_cast<const float*>(a.q) + qoff;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qo.q[kk] = live ? *reinterpret_cast<const float4*>(qp + 16 * kk + 4 * quad) : make_float4(0, 0, 0, 0);
    }
  }

  const size_t tile_elems = static_cast<size_t>(D) * BS;
  const size_t head_off = static_cast<size_t>(g) * tile_elems;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * tile_elems;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  constexpr size_t EB = BF16 ? 2 : 4;

  auto tile_ptrs = [&](int j, const void*& kt, const void*& vt) {
    int b = tbl[j];
    if (static_cast<unsigned>(b) >= static_cast<unsigned>(a.num_blocks)) b = 0;
    const size_t off = (static_cast<size_t>(b) * block_stride + head_off) * EB;
    kt = kbase + off;
    vt = vbase + off;
  };

  Acc<D> acc;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc.o[nt] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  constexpr int HALVES = BS / 16;
  Step<BF16, D> cur[HALVES], nxt[HALVES];

  int j = w;
  if (j < nblk) {
    const void *kt, *vt;
    tile_ptrs(j, kt, vt);
#pragma unroll
    for (int h = 0; h < HALVES; ++h) load_step<BF16, D, BS>(cur[h], kt, vt, h, row, quad);
  }
  for (; j < nblk; j += kWaves) {
    const int jn = j + kWaves;
    if (jn < nblk) {
      const void *kt, *vt;
      tile_ptrs(jn, kt, vt);
#pragma unroll
      for (int h = 0; h < HALVES; ++h) load_step<BF16, D, BS>(nxt[h], kt, vt, h, row, quad);
    }
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
      const int tok_base = start + j * BS + 16 * h;
      if (tok_base >= end) break;  // wave-uniform: the rest of the block is past the context
      Step<BF16, D>& st = cur[h];

      // Scores S[token 4*quad+i][head row] for the 16 tokens of this step.
      float4v sc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.k[kk]), qo.q[kk], sc, 0, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.k[kk].x, qo.q[kk].x, sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.k[kk].y, qo.q[kk].y, sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.k[kk].z, qo.q[kk].z, sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(st.k[kk].w, qo.q[kk].w, sc, 0, 0, 0);
        }
      }
      const bool tail = tok_base + 16 > end;  // wave-uniform
      const int tok0 = tok_base + 4 * quad;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sc[i] * a.scale_log2;
      if (tail) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + i >= end) x[i] = -INFINITY;
        mask_v<BF16, D>(st, tok0, end);
      }
      float bmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bmax = fmaxf(bmax, shfl_xor_f(bmax, 16));
      bmax = fmaxf(bmax, shfl_xor_f(bmax, 32));
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
      l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      if (__any(m_new > m_run)) {
        // Accumulator row r = 4*quad + v holds head (r mod 8) for bf16 (rows
        // 8..15 carry the low parts), head r for fp32; fetch its alpha.
        float av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int src = BF16 ? ((4 * quad + v) & 7) : (4 * quad + v);
          av[v] = __shfl(alpha, src, 64);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc.o[nt][v] *= av[v];
      }
      m_run = m_new;

      if constexpr (BF16) {
        short4v pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float other = row_rotate8(pr[i]);  // lanes 8..15 receive heads 0..7
          uint16_t bits;
          if (row < 8) {
            bits = f32_to_bf16_bits(pr[i]);
          } else {
            const uint16_t hi = f32_to_bf16_bits(other);
            bits = f32_to_bf16_bits(other - bf16_bits_to_f32(hi));
          }
          pa[i] = static_cast<short>(bits);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(short4v, st.v[nt]), acc.o[nt],
                                                                0, 0, 0);
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[0], st.v[nt].x, acc.o[nt], 0, 0, 0);
          acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[1], st.v[nt].y, acc.o[nt], 0, 0, 0);
          acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[2], st.v[nt].z, acc.o[nt], 0, 0, 0);
          acc.o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[3], st.v[nt].w, acc.o[nt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < HALVES; ++h) cur[h] = nxt[h];
  }

  // Per-wave totals: l over the four lane rows; bf16 high + low accumulator rows.
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if constexpr (BF16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc.o[nt][v] += shfl_xor_f(acc.o[nt][v], 32);
  }
  const int nw = nblk < kWaves ? nblk : kWaves;
  if (w < nw) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * quad + v;
      if (hh < G && (!BF16 || quad < 2)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm_o[w][hh][16 * nt + row] = acc.o[nt][v];
      }
    }
    if (quad == 0 && row < G) {
      sm_m[w][row] = m_run;
      sm_l[w][row] = l_run;
    }
  }
  __syncthreads();

  const size_t part_row0 = (static_cast<size_t>(s) * Hq + static_cast<size_t>(g) * G) * a.max_parts + p;
  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int hh = e / D;
    const int d = e - hh * D;
    float M = sm_m[0][hh];
    for (int ww = 1; ww < nw; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float num = 0.f, den = 0.f;
    for (int ww = 0; ww < nw; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm_m[ww][hh] - M);
      num += f * sm_o[ww][hh][d];
      den += f * sm_l[ww][hh];
    }
    if (nparts == 1) {
      const float o = num / den;
      if constexpr (BF16)
        static_cast<uint16_t*>(a.out)[out_row0 + e] = f32_to_bf16_bits(o);
      else
        static_cast<float*>(a.out)[out_row0 + e] = o;
    } else {
      const size_t pr0 = part_row0 + static_cast<size_t>(hh) * a.max_parts;
      a.ws_acc[pr0 * D + d] = num;
      if (d == 0) {
        a.ws_m[pr0] = M;
        a.ws_l[pr0] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partition partials of sequences with more than
// one partition.  One workgroup per (kv head, sequence) merges its G query
// heads: first the per-head maximum and weighted denominator over the
// partitions, then the weighted sum of the accumulator rows, read as
// coalesced 16-byte loads (one accumulator row is D contiguous floats).
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int GMAX = BF16 ? 8 : 16;
  __shared__ float sm_M[GMAX];
  __shared__ float sm_inv[GMAX];
  const int g = blockIdx.x;
  const int s = blockIdx.y;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
  const int P = a.partition_size;
  const int nparts = (L + P - 1) / P;
  if (nparts <= 1) return;
  const int G = a.group;
  const int mp = a.max_parts;
  const size_t head0 = static_cast<size_t>(s) * a.num_q_heads + static_cast<size_t>(g) * G;

  // Phase 1: per head, M = max_p m_p and den = sum_p 2^(m_p - M) l_p.
  // 16 threads per head (a quarter wave), strided over the partitions.
  {
    const int hh = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;
    for (int h0 = 0; h0 < G; h0 += kThreads / 16) {
      const int h = h0 + hh;
      const bool live = h < G;
      const float* mrow = a.ws_m + (head0 + (live ? h : 0)) * mp;
      const float* lrow = a.ws_l + (head0 + (live ? h : 0)) * mp;
      float M = -INFINITY;
      if (live)
        for (int p = sub; p < nparts; p += 16) M = fmaxf(M, mrow[p]);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 16));
      float den = 0.f;
      if (live)
        for (int p = sub; p < nparts; p += 16) den += __builtin_amdgcn_exp2f(mrow[p] - M) * lrow[p];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) den += __shfl_xor(den, off, 16);
      if (live && sub == 0) {
        sm_M[h] = M;
        sm_inv[h] = 1.f / den;
      }
    }
  }
  __syncthreads();

  // Phase 2: each thread owns 4 consecutive dims of one head.
  for (int e = threadIdx.x * 4; e < G * D; e += kThreads * 4) {
    const int h = e / D;
    const int d = e - h * D;
    const float M = sm_M[h];
    const float* mrow = a.ws_m + (head0 + h) * mp;
    const float* arow = a.ws_acc + (head0 + h) * mp * D + d;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int p = 0;
    for (; p + 4 <= nparts; p += 4) {
      float4 v[4];
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = *reinterpret_cast<const float4*>(arow + static_cast<size_t>(p + i) * D);
        f[i] = __builtin_amdgcn_exp2f(mrow[p + i] - M);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc.x += f[i] * v[i].x;
        acc.y += f[i] * v[i].y;
        acc.z += f[i] * v[i].z;
        acc.w += f[i] * v[i].w;
      }
    }
    for (; p < nparts; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(arow + static_cast<size_t>(p) * D);
      const float f = __builtin_amdgcn_exp2f(mrow[p] - M);
      acc.x += f * v.x;
      acc.y += f * v.y;
      acc.z += f * v.z;
      acc.w += f * v.w;
    }
    const float inv = sm_inv[h];
    const size_t o = (head0 + h) * D + d;
    const float r[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BF16)
        static_cast<uint16_t*>(a.out)[o + i] = f32_to_bf16_bits(r[i]);
      else
        static_cast<float*>(a.out)[o + i] = r[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Cache append: one thread per (token, kv head, 16-byte chunk of head_dim).
template <int EB>
__global__ __launch_bounds__(256) void append_kernel(const char* __restrict__ k_new, const char* __restrict__ v_new,
                                                     char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                     const int32_t* __restrict__ slot_mapping, int64_t total,
                                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                     int32_t num_blocks) {
  constexpr int X = 16 / EB;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int nch = head_dim / X;
  const int c = static_cast<int>(idx % nch);
  const int64_t th = idx / nch;
  const int h = static_cast<int>(th % num_kv_heads);
  const int64_t t = th / num_kv_heads;
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(num_blocks) * block_size) return;
  const int64_t b = slot / block_size;
  const int o = slot - static_cast<int32_t>(b) * block_size;
  const int64_t src = ((t * num_kv_heads + h) * head_dim + static_cast<int64_t>(c) * X) * EB;
  const uint4 kv = *reinterpret_cast<const uint4*>(k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(v_new + src);
  const int64_t tile = (b * num_kv_heads + h) * static_cast<int64_t>(head_dim) * block_size;
  *reinterpret_cast<uint4*>(k_cache + ((tile + (static_cast<int64_t>(c) * block_size + o) * X) * EB)) = kv;
  const int64_t vdst = tile + static_cast<int64_t>(c) * X * block_size + o;
  if constexpr (EB == 2) {
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
    uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache);
#pragma unroll
    for (int i = 0; i < 8; ++i) vc[vdst + static_cast<int64_t>(i) * block_size] = static_cast<uint16_t>(w[i / 2] >> (16 * (i & 1)));
  } else {
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
    uint32_t* vc = reinterpret_cast<uint32_t*>(v_cache);
#pragma unroll
    for (int i = 0; i < 4; ++i) vc[vdst + static_cast<int64_t>(i) * block_size] = w[i];
  }
}

// Block copy: blockIdx.x = pair, blockIdx.y = 0 (K pool) or 1 (V pool).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                          const int32_t* __restrict__ src_dst, int64_t block_bytes,
                                                          int32_t num_blocks) {
  const int pair = blockIdx.x;
  const int32_t src = src_dst[2 * pair];
  const int32_t dst = src_dst[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* pool = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* from = reinterpret_cast<const uint4*>(pool + static_cast<int64_t>(src) * block_bytes);
  uint4* to = reinterpret_cast<uint4*>(pool + static_cast<int64_t>(dst) * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) to[i] = from[i];
}

// ---------------------------------------------------------------------------
int32_t check_common(int32_t head_dim, int32_t block_size, pkv_dtype dt) {
  if (dt != PKV_F32 && dt != PKV_BF16) return pkv::fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
  if (head_dim != 64 && head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported (16 or 32)", block_size);
  return PKV_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return pkv::ok();
}

// Default partition: enough (sequence, kv head, partition) workgroups to
// fill the chip several times over (about 2048), in power-of-two token
// counts between 256 and 2048.  The upper bound keeps one workgroup's share
// of a long context short enough that a batch of mixed lengths does not end
// on a few long workgroups; the 32k layer measures best at 2048.
constexpr int64_t kTargetWorkgroups = 2048;
constexpr int32_t kMinPartition = 256;
constexpr int32_t kMaxPartition = 2048;

int32_t default_partition(int64_t num_seqs, int64_t num_kv_heads, int64_t max_context_len, int32_t block_size) {
  const int64_t pairs = num_seqs * num_kv_heads > 0 ? num_seqs * num_kv_heads : 1;
  const int64_t parts = (kTargetWorkgroups + pairs - 1) / pairs;
  const int64_t want = (max_context_len + parts - 1) / parts;
  int32_t P = kMinPartition;
  while (P < kMaxPartition && P < want) P *= 2;
  return P < block_size ? block_size : P;
}

int32_t resolve_partition(int32_t partition_size, int32_t block_size, int64_t num_seqs, int64_t num_kv_heads,
                          int64_t max_context_len, int32_t* out) {
  int32_t P = partition_size == 0 ? default_partition(num_seqs, num_kv_heads, max_context_len, block_size)
                                  : partition_size;
  if (P <= 0 || P % block_size)
    return pkv::fail(PKV_ERR_INVALID_ARG, "partition_size %d must be a positive multiple of block_size %d", P,
                     block_size);
  *out = P;
  return PKV_OK;
}

size_t workspace_for(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim, int64_t max_parts) {
  if (max_parts <= 1) return 0;
  const int64_t rows = num_seqs * num_q_heads * max_parts;
  const int64_t acc = ((rows * head_dim * 4 + 255) / 256) * 256;
  const int64_t ml = ((rows * 4 + 255) / 256) * 256;
  return static_cast<size_t>(acc + 2 * ml);
}

template <bool BF16, int D, int BS>
void launch_decode(const DecodeArgs& a, int32_t num_seqs, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_kv_heads, num_seqs);
  decode_partition_kernel<BF16, D, BS><<<grid, kThreads, 0, st>>>(a);
  if (a.max_parts > 1) decode_merge_kernel<BF16, D><<<dim3(a.num_kv_heads, num_seqs), kThreads, 0, st>>>(a);
}

template <bool BF16, int D>
void dispatch_bs(const DecodeArgs& a, int32_t num_seqs, int32_t bs, hipStream_t st) {
  if (bs == 16)
    launch_decode<BF16, D, 16>(a, num_seqs, st);
  else
    launch_decode<BF16, D, 32>(a, num_seqs, st);
}

}  // namespace

namespace pkv {
std::string& last_error_slot() {
  thread_local std::string msg;
  return msg;
}
}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return pkv::last_error_slot().c_str(); }

int32_t pkv_version(void) { return 100; }

int32_t paged_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t num_blocks, pkv_dtype dt, void* stream) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes: num_tokens %d num_kv_heads %d num_blocks %d", num_tokens,
                     num_kv_heads, num_blocks);
  if (num_tokens == 0) return pkv::ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  const int eb = dt == PKV_BF16 ? 2 : 4;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim * eb / 16);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "too many tokens for one launch");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (eb == 2)
    append_kernel<2><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, st>>>(
        static_cast<const char*>(k_new), static_cast<const char*>(v_new), static_cast<char*>(k_cache),
        static_cast<char*>(v_cache), slot_mapping, total, num_kv_heads, head_dim, block_size, num_blocks);
  else
    append_kernel<4><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, st>>>(
        static_cast<const char*>(k_new), static_cast<const char*>(v_new), static_cast<char*>(k_cache),
        static_cast<char*>(v_cache), slot_mapping, total, num_kv_heads, head_dim, block_size, num_blocks);
  return launch_status("paged_kv_append");
}

int32_t paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t num_pairs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             pkv_dtype dt, void* stream) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes: num_pairs %d num_kv_heads %d num_blocks %d", num_pairs,
                     num_kv_heads, num_blocks);
  if (num_pairs == 0) return pkv::ok();
  if (!k_cache || !v_cache || !src_dst) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID_ARG, "K/V pools must be 16-byte aligned");
  const int eb = dt == PKV_BF16 ? 2 : 4;
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * eb;
  copy_blocks_kernel<<<dim3(num_pairs, 2), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<char*>(k_cache), static_cast<char*>(v_cache), src_dst, block_bytes, num_blocks);
  return launch_status("paged_kv_copy_blocks");
}

int32_t paged_attention_default_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_context_len) {
  if (int32_t e = check_common(head_dim, block_size, PKV_BF16)) return e;
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes");
  int32_t P = 0;
  if (int32_t e = resolve_partition(0, block_size, num_seqs, num_kv_heads, max_context_len, &P)) return e;
  pkv::ok();
  return P;
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_context_len, int32_t partition_size) {
  if (check_common(head_dim, block_size, PKV_BF16)) return 0;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) {
    pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes");
    return 0;
  }
  int32_t P = 0;
  if (resolve_partition(partition_size, block_size, num_seqs, num_kv_heads, max_context_len, &P)) return 0;
  const int64_t max_parts = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  pkv::ok();
  return workspace_for(num_seqs, num_q_heads, head_dim, max_parts);
}

int32_t paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dt,
                               void* stream) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "bad sizes: num_seqs %d num_q_heads %d num_kv_heads %d num_blocks %d max_blocks_per_seq %d "
                     "max_context_len %d",
                     num_seqs, num_q_heads, num_kv_heads, num_blocks, max_blocks_per_seq, max_context_len);
  if (num_q_heads % num_kv_heads)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                     num_kv_heads);
  const int32_t G = num_q_heads / num_kv_heads;
  const int32_t gmax = dt == PKV_BF16 ? 8 : 16;
  if (G > gmax) return pkv::fail(PKV_ERR_UNSUPPORTED, "query group size %d > %d not supported", G, gmax);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks_per_seq * block_size", max_context_len);
  if (num_seqs > 65535 || num_kv_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs and num_kv_heads must be <= 65535");
  if (!std::isfinite(scale)) return pkv::fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (num_seqs == 0) return pkv::ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID_ARG, "q, out and the pools must be 16-byte aligned");
  int32_t P = 0;
  if (int32_t e = resolve_partition(partition_size, block_size, num_seqs, num_kv_heads, max_context_len, &P))
    return e;
  const int64_t max_parts = max_context_len == 0 ? 1 : (static_cast<int64_t>(max_context_len) + P - 1) / P;
  if (max_parts > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "too many partitions");
  const size_t need = workspace_for(num_seqs, num_q_heads, head_dim, max_parts);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return pkv::fail(PKV_ERR_CAPACITY, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return pkv::fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * max_parts;
  char* ws = static_cast<char*>(workspace);
  const int64_t acc_bytes = ((rows * head_dim * 4 + 255) / 256) * 256;
  const int64_t ml_bytes = ((rows * 4 + 255) / 256) * 256;
  a.ws_acc = need ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_m = need ? reinterpret_cast<float*>(ws + acc_bytes) : nullptr;
  a.ws_l = need ? reinterpret_cast<float*>(ws + acc_bytes + ml_bytes) : nullptr;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.partition_size = P;
  a.max_parts = static_cast<int32_t>(max_parts);
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == PKV_BF16) {
    if (head_dim == 128)
      dispatch_bs<true, 128>(a, num_seqs, block_size, st);
    else
      dispatch_bs<true, 64>(a, num_seqs, block_size, st);
  } else {
    if (head_dim == 128)
      dispatch_bs<false, 128>(a, num_seqs, block_size, st);
    else
      dispatch_bs<false, 64>(a, num_seqs, block_size, st);
  }
  return launch_status("paged_attention_decode");
}

}  // extern "C"
