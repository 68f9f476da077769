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
//   * A decode step's one-token cache append (step 3 of the aitalk page)
//     can ride along: the workgroup that reads a sequence's last block
//     first writes the new K/V row into it (a workgroup whose range holds
//     the ends of several short sequences writes one row per segment).
//     This is done only when there are at most as many sequences as
//     workgroups per kv head; otherwise a small append kernel runs first.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "pkv_status.h"

// 1 builds the A/B library whose bf16 decode products run on the vector ALUs
// (decode_segment_valu); the product library is built with 0.
#ifndef PKV_DECODE_VALU_DOT
#define PKV_DECODE_VALU_DOT 0
#endif

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(4))) float float4v;
// plain vector types for the non-temporal load builtin
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4v;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2v;
typedef __attribute__((ext_vector_type(4))) float f32x4v;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Block ids of a segment are staged in LDS this many at a time, so the step
// loop reads them with LDS loads (ordered by lgkmcnt) rather than vector
// memory loads, whose in-order completion counter would make each table read
// wait for the K/V loads still in flight.
constexpr int kIdChunk = 1024;

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

// Device status word (one per GPU): kernels OR a PKV_DEV_* flag into it when
// they meet a device-side index outside its range (the offending access is
// skipped or clamped into the buffers).  pkv_device_status reads and clears it.
__device__ __forceinline__ void report(int32_t* status, int32_t flag) {
  __hip_atomic_fetch_or(status, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;  // [S][Hkv][D] token appended at position L - 1, or null
  const void* v_new;
  float* ws_acc;     // [N][2][G][D] partial accumulators (workgroup, slot, head)
  float* ws_m;       // [N][2][G] partial max (log2 domain)
  float* ws_l;       // [N][2][G] partial sum
  int32_t* meta;     // [S][Hkv][2] first workgroup index and number of pieces of (s, g)
  int32_t* status;   // device status word
  int32_t wgs_per_head;  // N / Hkv
  int32_t seg_cost;      // fixed cost of one segment in the balanced split, in blocks
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
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
//
// Cache policy (SH: the call's flags say that several sequences read the
// same blocks).  Without sharing, each K/V byte is read once per call, so
// the loads are non-temporal (the `nt` policy): a plain load also
// allocates each streamed line in the 256 MB Infinity Cache, and with
// gigabytes streaming through that costs bandwidth (the 16 x 32k layer's
// decode call took 335 instead of 374 us).  The exception is V at block
// size 32: one dimension's V row is 64 bytes, a 16-token unit reads half of
// it and the partner wave reads the other half, which then has to be found
// in cache; there V loads are plain (with non-temporal V the mixed-length
// bs32 batch was 10 % slower, with plain V and non-temporal K 6 % faster
// than all plain).  With sharing (prefix caching, forked samples) a block
// fetched for one sequence should serve the others from cache, so every
// load is plain (the 400 forked samples of 50 prompts: 234 against 285 us).
template <typename T, typename V>
__device__ __forceinline__ T load_nt(const T* p) {
  return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const V*>(p)));
}

template <bool BF16, int D, int BS, bool SH>
__device__ __forceinline__ void load_step(Step<BF16, D>& st, const void* k_tile, const void* v_tile, int h, int row,
                                          int quad) {
  constexpr bool kKnt = !SH;
  constexpr bool kVnt = !SH && BS == 16;  // a unit reads whole V rows
  if constexpr (BF16) {
    const uint16_t* kt = static_cast<const uint16_t*>(k_tile);
    const uint16_t* vt = static_cast<const uint16_t*>(v_tile);
#pragma unroll
    for (int kk = 0; kk < Step<BF16, D>::KK; ++kk)
    {
      const uint4* p = reinterpret_cast<const uint4*>(kt + ((4 * kk + quad) * BS + 16 * h + row) * 8);
      st.k[kk] = kKnt ? load_nt<uint4, u32x4v>(p) : *p;
    }
#pragma unroll
    for (int nt = 0; nt < Step<BF16, D>::NT; ++nt) {
      const uint2* p = reinterpret_cast<const uint2*>(vt + (16 * nt + row) * BS + 16 * h + 4 * quad);
      st.v[nt] = kVnt ? load_nt<uint2, u32x2v>(p) : *p;
    }
  } else {
    const float* kt = static_cast<const float*>(k_tile);
    const float* vt = static_cast<const float*>(v_tile);
#pragma unroll
    for (int kk = 0; kk < Step<BF16, D>::KK; ++kk)
    {
      const float4* p = reinterpret_cast<const float4*>(kt + ((4 * kk + quad) * BS + 16 * h + row) * 4);
      st.k[kk] = kKnt ? load_nt<float4, f32x4v>(p) : *p;
    }
#pragma unroll
    for (int nt = 0; nt < Step<BF16, D>::NT; ++nt) {
      const float4* p = reinterpret_cast<const float4*>(vt + (16 * nt + row) * BS + 16 * h + 4 * quad);
      st.v[nt] = kVnt ? load_nt<float4, f32x4v>(p) : *p;
    }
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

template <bool BF16, int D>
struct DecodeSmem {
  static constexpr int GMAX = BF16 ? 8 : 16;
  float o[kWaves][GMAX][D];  // per-wave accumulators of the current segment
  float m[kWaves][GMAX];
  float l[kWaves][GMAX];
  int wave_sum[kWaves];
  int found_seq;
  int found_pre;
  // k_new / v_new of an appending call, parked here so the kernel does not
  // hold them in scalar registers through the step loop
  const void* append_src[2];
  int ids[kIdChunk];  // block ids of the current chunk of the segment
  int lens[kThreads];  // raw context lengths, when the batch has at most kThreads sequences
#if PKV_DECODE_VALU_DOT
  uint16_t qv[8][D];          // the group's query rows (bf16), zero past G
  float pv[kWaves][16][8];    // one unit's probabilities, [token][head], per wave
#endif
};

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }

// Inclusive prefix sum of one int per thread over the workgroup; *total
// receives the workgroup total.  All threads must call it.
template <bool BF16, int D>
__device__ __forceinline__ int block_scan(int v, int* total, DecodeSmem<BF16, D>& sm) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sm.wave_sum[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += i < w ? sm.wave_sum[i] : 0;
    tot += sm.wave_sum[i];
  }
  __syncthreads();
  *total = tot;
  return before + x;
}

// Partial row of (workgroup b, slot) for head hh: ((b * 2 + slot) * G + hh).
// Slot 1 holds a piece that starts at its sequence's first block, slot 0 a
// piece that starts inside the sequence.

// The cache append done by the decode kernel: the K/V row of kv head g of
// the token at position L - 1 of sequence s, from k_new/v_new
// [S][Hkv][D], goes into its pool slot, written by the workgroup that
// reads that slot.  The tile formats are those of the pools: K
// [D/X][BS][X] (X = 16 bytes of elements), V [D][BS].  A block id outside
// the pool skips the write.  The loads (table entry, one K chunk or one V
// element per thread) are independent and issued together with the staging
// of the segment's block ids, so they add no round trip of their own.
template <bool BF16, int D>
struct AppendRow {
  uint4 k;     // K chunk `threadIdx.x` (threads < D / X)
  uint32_t v;  // V element `threadIdx.x` (threads < D)
  int32_t blk;
};

template <bool BF16, int D, int BS>
__device__ __forceinline__ AppendRow<BF16, D> append_load(const DecodeArgs& a, const void* k_new, const void* v_new,
                                                          int s, int g, int L) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int X = 16 / EB;
  static_assert(D <= kThreads, "one V element per thread");
  AppendRow<BF16, D> r;
  r.blk = a.block_tables[static_cast<size_t>(s) * a.max_blocks_per_seq + (L - 1) / BS];
  const size_t src = (static_cast<size_t>(s) * a.num_kv_heads + g) * D;
  const int t = threadIdx.x;
  r.k = make_uint4(0, 0, 0, 0);
  r.v = 0;
  if (t < D / X) r.k = *reinterpret_cast<const uint4*>(static_cast<const char*>(k_new) + (src + t * X) * EB);
  if (t < D) {
    if constexpr (BF16)
      r.v = static_cast<const uint16_t*>(v_new)[src + t];
    else
      r.v = static_cast<const uint32_t*>(v_new)[src + t];
  }
  return r;
}

template <bool BF16, int D, int BS>
__device__ __forceinline__ void append_store(const DecodeArgs& a, const AppendRow<BF16, D>& r, int g, int L) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int X = 16 / EB;
  if (static_cast<unsigned>(r.blk) >= static_cast<unsigned>(a.num_blocks)) {
    if (threadIdx.x == 0) report(a.status, PKV_DEV_BAD_BLOCK_ID);
    return;
  }
  const int o = (L - 1) % BS;
  const size_t tile = (static_cast<size_t>(r.blk) * a.num_kv_heads + g) * static_cast<size_t>(D) * BS;
  char* kc = const_cast<char*>(static_cast<const char*>(a.k_cache));
  char* vc = const_cast<char*>(static_cast<const char*>(a.v_cache));
  const int t = threadIdx.x;
  if (t < D / X) *reinterpret_cast<uint4*>(kc + (tile + (static_cast<size_t>(t) * BS + o) * X) * EB) = r.k;
  if (t < D) {
    if constexpr (BF16)
      reinterpret_cast<uint16_t*>(vc)[tile + static_cast<size_t>(t) * BS + o] = static_cast<uint16_t>(r.v);
    else
      reinterpret_cast<uint32_t*>(vc)[tile + static_cast<size_t>(t) * BS + o] = r.v;
  }
}

// The end of a segment: waves w < nw have left their (max, sum,
// accumulator) in sm.m/l/o; they are combined, and the output rows (prow <
// 0) or partial row `prow` written.
template <bool BF16, int D>
__device__ __forceinline__ void merge_waves(const DecodeArgs& a, DecodeSmem<BF16, D>& sm, int nw, int prow,
                                            size_t out_row0) {
  const int G = a.group;
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int hh = e / D;
    const int d = e - hh * D;
    float M = sm.m[0][hh];
    for (int ww = 1; ww < nw; ++ww) M = fmaxf(M, sm.m[ww][hh]);
    float num = 0.f, den = 0.f;
    for (int ww = 0; ww < nw; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm.m[ww][hh] - M);
      num += f * sm.o[ww][hh][d];
      den += f * sm.l[ww][hh];
    }
    if (prow < 0) {
      const float o = num / den;
      if constexpr (BF16)
        static_cast<uint16_t*>(a.out)[out_row0 + e] = f32_to_bf16_bits(o);
      else
        static_cast<float*>(a.out)[out_row0 + e] = o;
    } else {
      const size_t r = static_cast<size_t>(prow) * G + hh;
      a.ws_acc[r * D + d] = num;
      if (d == 0) {
        a.ws_m[r] = M;
        a.ws_l[r] = den;
      }
    }
  }
  __syncthreads();  // the next segment reuses the LDS
}

// Blocks [lb0, lb1) of sequence s (length L) for kv head g.  When
// `prow` < 0 the segment is the whole sequence and the output rows are
// written; otherwise (max, sum, accumulator) go to partial row `prow`.
// With `append`, the segment holds the sequence's last block and first
// writes the appended token's K/V into it; the workgroup barrier after the
// staging of the block ids orders those stores before every wave's loads
// of the block (one workgroup: one compute unit and its L1).
template <bool BF16, int D, int BS, bool SH>
__device__ void decode_segment(const DecodeArgs& a, int s, int g, int L, int lb0, int lb1, int prow, bool append,
                               DecodeSmem<BF16, D>& sm) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int quad = lane >> 4;
  const int G = a.group;
  const int Hq = a.num_q_heads;

  const int start = lb0 * BS;
  const int end = min(lb1 * BS, L);
  const int nblk = lb1 - lb0;
  const int32_t* tbl = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq + lb0;
  const size_t out_row0 = (static_cast<size_t>(s) * Hq + static_cast<size_t>(g) * G) * D;

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

  // Tile pointers of chunk-local block c (block id from LDS, made scalar).
  auto tile_ptrs = [&](int c, const void*& kt, const void*& vt) {
    const int b = __builtin_amdgcn_readfirstlane(sm.ids[c]);
    const size_t off = (static_cast<size_t>(b) * block_stride + head_off) * EB;
    kt = kbase + off;
    vt = vbase + off;
  };

  Acc<D> acc;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc.o[nt] = float4v{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto compute_step = [&](Step<BF16, D>& st, const int tok_base) {

      // Scores S[token 4*quad+i][head row] for the 16 tokens of this step.
      // bf16: the dot product runs as two chained halves (dims 0..D/2-1
      // and D/2..D-1), whose results are summed without rounding error into
      // sc + sl (Knuth's two-sum), so the score carries only the halves' own
      // roundings.  With logits in the hundreds, rounding every partial sum
      // of one chained product to fp32 moves the softmax weights of
      // near-tied keys enough to show in outputs near zero.
      float4v sc = {0.f, 0.f, 0.f, 0.f};
      float4v sl = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        constexpr int KK = D / 32;
        float4v half_sum[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
  #pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          half_sum[kk / (KK / 2)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, st.k[kk]), qo.q[kk], half_sum[kk / (KK / 2)], 0, 0, 0);
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = half_sum[0][i], b0 = half_sum[1][i];
          const float s0 = a0 + b0;
          const float bv = s0 - a0;
          sl[i] = (a0 - (s0 - bv)) + (b0 - bv);
          sc[i] = s0;
        }
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
      if constexpr (BF16) {
        // exponent (sc + sl) * scale - m with the large terms in one fused
        // operation: only the small remainder is rounded
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fmaf(sc[i], a.scale_log2, -m_new) + sl[i] * a.scale_log2;
          pr[i] = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(e);
        }
      } else {
  #pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
      }
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
  };

  // The segment's tokens are cut into 16-token units (two per block when
  // BS = 32) dealt to the waves round robin: wave w takes units w, w + 4,
  // ..., loading unit n+1 while computing unit n.  With BS = 32 the two
  // halves of a block go to waves 2i and 2i+1, which load them at about the
  // same time; a 64-byte V row (one dimension, 32 tokens) is then read by
  // both halves together, not by one wave a whole step after the other,
  // which in a saturated stream lets the line leave L2 in between and be
  // fetched again.  Block ids come through LDS, kIdChunk at a time.
  constexpr int HALVES = BS / 16;
  static_assert(kWaves % HALVES == 0, "a wave keeps the same half of every block it visits");
  const int h = w % HALVES;
  const int nunits = (end - start + 15) / 16;
  auto stage_ids = [&](int c0) {
    const int cn = nblk - c0 < kIdChunk ? nblk - c0 : kIdChunk;
    for (int i = threadIdx.x; i < cn; i += kThreads) {
      const int b = tbl[c0 + i];
      const bool ok = static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks);
      if (!ok) report(a.status, PKV_DEV_BAD_BLOCK_ID);
      sm.ids[i] = ok ? b : 0;
    }
  };
  // The first chunk's ids are staged before the loop, so the append (its
  // loads issued with them, its stores after) ends before the step loop.
  if (append) {
    const void* kn = sm.append_src[0];
    const void* vn = sm.append_src[1];
    const AppendRow<BF16, D> arow = append_load<BF16, D, BS>(a, kn, vn, s, g, L);
    stage_ids(0);
    append_store<BF16, D, BS>(a, arow, g, L);
  } else {
    stage_ids(0);
  }
  for (int c0 = 0; c0 < nblk; c0 += kIdChunk) {
    const int cn = nblk - c0 < kIdChunk ? nblk - c0 : kIdChunk;
    if (c0 > 0) stage_ids(c0);
    __syncthreads();
    // units [c0 * HALVES, uend) lie in this chunk's blocks; each holds at
    // least one valid token
    const int uend = c0 * HALVES + (min(start + (c0 + cn) * BS, end) - (start + c0 * BS) + 15) / 16;
    Step<BF16, D> st, nxt;
    const void* kt = nullptr;
    const void* vt = nullptr;
    int u = c0 * HALVES + w;
    if (u < uend) {
      tile_ptrs(u / HALVES - c0, kt, vt);
      load_step<BF16, D, BS, SH>(st, kt, vt, h, row, quad);
      // Every loop trip issues the next unit's loads unconditionally, so the
      // wait before the current unit's math covers only its own loads; the
      // last unit runs after the loop.
      for (;;) {
        const int un = u + kWaves;
        if (un >= uend) break;
        tile_ptrs(un / HALVES - c0, kt, vt);
        load_step<BF16, D, BS, SH>(nxt, kt, vt, h, row, quad);
        compute_step(st, start + 16 * u);
        st = nxt;
        u = un;
      }
      compute_step(st, start + 16 * u);
    }
    __syncthreads();  // sm.ids is rewritten by the next chunk
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
  const int nw = nunits < kWaves ? nunits : kWaves;  // waves that took at least one unit
  if (w < nw) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 4 * quad + v;
      if (hh < G && (!BF16 || quad < 2)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm.o[w][hh][16 * nt + row] = acc.o[nt][v];
      }
    }
    if (quad == 0 && row < G) {
      sm.m[w][row] = m_run;
      sm.l[w][row] = l_run;
    }
  }
  merge_waves<BF16, D>(a, sm, nw, prow, out_row0);
}

#if PKV_DECODE_VALU_DOT
// Vector-ALU variant of the bf16 segment, built only into the A/B library
// that measures what the matrix cores buy (the product library always uses
// decode_segment).  Same loads, unit walk, online softmax and merge; the
// products run on the VALU:
//   * Q.K: lane (row, quad) holds 32 dims of token `row` (as loaded for the
//     MFMA); it takes the same dims of each of the GV query heads from LDS
//     and accumulates v_dot2_f32_bf16 (two bf16 products per instruction)
//     in two chains, then the four quads' partial dots are summed by
//     shuffles: every lane ends with the scores of its token for all heads.
//   * P.V: each wave writes its unit's probabilities to LDS; lane (row,
//     quad) reads those of tokens 4 quad .. 4 quad + 3 and accumulates, in
//     fp32 FMAs, dims 16 nt + row of all GV heads over its four tokens; the
//     quads' partial sums are added at the end of the segment.
// GV (4 or 8) is the compile-time head count the loops run over.
template <int D, int BS, int GV, bool SH>
__device__ void decode_segment_valu(const DecodeArgs& a, int s, int g, int L, int lb0, int lb1, int prow,
                                    bool append, DecodeSmem<true, D>& sm) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  constexpr int NT = D / 16;
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int quad = lane >> 4;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int start = lb0 * BS;
  const int end = min(lb1 * BS, L);
  const int nblk = lb1 - lb0;
  const int32_t* tbl = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq + lb0;
  const size_t out_row0 = (static_cast<size_t>(s) * Hq + static_cast<size_t>(g) * G) * D;

  // the group's query rows into LDS (ordered before use by the barrier
  // after the block-id staging)
  for (int e = threadIdx.x; e < GV * D; e += kThreads) {
    const int hh = e / D;
    sm.qv[hh][e - hh * D] = hh < G ? static_cast<const uint16_t*>(a.q)[out_row0 + e] : uint16_t{0};
  }

  const size_t tile_elems = static_cast<size_t>(D) * BS;
  const size_t head_off = static_cast<size_t>(g) * tile_elems;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * tile_elems;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  auto tile_ptrs = [&](int c, const void*& kt, const void*& vt) {
    const int b = __builtin_amdgcn_readfirstlane(sm.ids[c]);
    const size_t off = (static_cast<size_t>(b) * block_stride + head_off) * 2;
    kt = kbase + off;
    vt = vbase + off;
  };

  float acc[NT][GV];
  float m_run[GV], l_run[GV];
#pragma unroll
  for (int h = 0; h < GV; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt][h] = 0.f;
  }

  auto compute_step = [&](Step<true, D>& st, const int tok_base) {
    float x[GV];
    const bool valid = tok_base + row < end;
#pragma unroll
    for (int h = 0; h < GV; ++h) {
      float c0 = 0.f, c1 = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 qq = *reinterpret_cast<const uint4*>(&sm.qv[h][8 * (4 * kk + quad)]);
        const uint4 kv = st.k[kk];
        c0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv.x), __builtin_bit_cast(bf16x2, qq.x), c0,
                                             false);
        c1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv.y), __builtin_bit_cast(bf16x2, qq.y), c1,
                                             false);
        c0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv.z), __builtin_bit_cast(bf16x2, qq.z), c0,
                                             false);
        c1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kv.w), __builtin_bit_cast(bf16x2, qq.w), c1,
                                             false);
      }
      float t = c0 + c1;
      t += shfl_xor_f(t, 16);
      t += shfl_xor_f(t, 32);
      x[h] = valid ? t * a.scale_log2 : -INFINITY;
    }
    if (tok_base + 16 > end) mask_v<true, D>(st, tok_base + 4 * quad, end);
    float p[GV], alpha[GV];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < GV; ++h) {
      float bm = x[h];
      bm = fmaxf(bm, shfl_xor_f(bm, 1));
      bm = fmaxf(bm, shfl_xor_f(bm, 2));
      bm = fmaxf(bm, shfl_xor_f(bm, 4));
      bm = fmaxf(bm, shfl_xor_f(bm, 8));
      const float m_new = fmaxf(m_run[h], bm);
      alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      grow |= m_new > m_run[h];
      p[h] = valid ? __builtin_amdgcn_exp2f(x[h] - m_new) : 0.f;
      l_run[h] = l_run[h] * alpha[h] + p[h];
      m_run[h] = m_new;
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < GV; ++h) acc[nt][h] *= alpha[h];
    }
    if (quad == 0) {
#pragma unroll
      for (int h = 0; h < GV; ++h) sm.pv[w][row][h] = p[h];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pt[4][GV];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < GV; ++h) pt[i][h] = sm.pv[w][4 * quad + i][h];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float v0 = bf16_bits_to_f32(static_cast<uint16_t>(st.v[nt].x & 0xFFFFu));
      const float v1 = bf16_bits_to_f32(static_cast<uint16_t>(st.v[nt].x >> 16));
      const float v2 = bf16_bits_to_f32(static_cast<uint16_t>(st.v[nt].y & 0xFFFFu));
      const float v3 = bf16_bits_to_f32(static_cast<uint16_t>(st.v[nt].y >> 16));
#pragma unroll
      for (int h = 0; h < GV; ++h)
        acc[nt][h] = fmaf(pt[3][h], v3, fmaf(pt[2][h], v2, fmaf(pt[1][h], v1, fmaf(pt[0][h], v0, acc[nt][h]))));
    }
    // the next unit's stores to sm.pv come after every lane's reads above
    __builtin_amdgcn_wave_barrier();
  };

  constexpr int HALVES = BS / 16;
  const int h = w % HALVES;
  const int nunits = (end - start + 15) / 16;
  auto stage_ids = [&](int c0) {
    const int cn = nblk - c0 < kIdChunk ? nblk - c0 : kIdChunk;
    for (int i = threadIdx.x; i < cn; i += kThreads) {
      const int b = tbl[c0 + i];
      const bool ok = static_cast<unsigned>(b) < static_cast<unsigned>(a.num_blocks);
      if (!ok) report(a.status, PKV_DEV_BAD_BLOCK_ID);
      sm.ids[i] = ok ? b : 0;
    }
  };
  if (append) {
    const AppendRow<true, D> arow = append_load<true, D, BS>(a, sm.append_src[0], sm.append_src[1], s, g, L);
    stage_ids(0);
    append_store<true, D, BS>(a, arow, g, L);
  } else {
    stage_ids(0);
  }
  for (int c0 = 0; c0 < nblk; c0 += kIdChunk) {
    const int cn = nblk - c0 < kIdChunk ? nblk - c0 : kIdChunk;
    if (c0 > 0) stage_ids(c0);
    __syncthreads();
    const int uend = c0 * HALVES + (min(start + (c0 + cn) * BS, end) - (start + c0 * BS) + 15) / 16;
    Step<true, D> st, nxt;
    const void* kt = nullptr;
    const void* vt = nullptr;
    int u = c0 * HALVES + w;
    if (u < uend) {
      tile_ptrs(u / HALVES - c0, kt, vt);
      load_step<true, D, BS, SH>(st, kt, vt, h, row, quad);
      for (;;) {
        const int un = u + kWaves;
        if (un >= uend) break;
        tile_ptrs(un / HALVES - c0, kt, vt);
        load_step<true, D, BS, SH>(nxt, kt, vt, h, row, quad);
        compute_step(st, start + 16 * u);
        st = nxt;
        u = un;
      }
      compute_step(st, start + 16 * u);
    }
    __syncthreads();
  }

  // per-wave totals: l over the 16 token rows, accumulators over the quads
#pragma unroll
  for (int hh = 0; hh < GV; ++hh) {
    float t = l_run[hh];
    t += shfl_xor_f(t, 1);
    t += shfl_xor_f(t, 2);
    t += shfl_xor_f(t, 4);
    t += shfl_xor_f(t, 8);
    l_run[hh] = t;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt][hh] += shfl_xor_f(acc[nt][hh], 16);
      acc[nt][hh] += shfl_xor_f(acc[nt][hh], 32);
    }
  }
  const int nw = nunits < kWaves ? nunits : kWaves;
  if (w < nw && quad == 0) {
#pragma unroll
    for (int hh = 0; hh < GV; ++hh) {
      if (hh < G) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm.o[w][hh][16 * nt + row] = acc[nt][hh];
        if (row == 0) {
          sm.m[w][hh] = m_run[hh];
          sm.l[w][hh] = l_run[hh];
        }
      }
    }
  }
  merge_waves<true, D>(a, sm, nw, prow, out_row0);
}
#endif

// Balanced split.  For one kv head, the blocks of all sequences form one
// list (sequence after sequence) in which every non-empty sequence is also
// charged seg_cost blocks' worth of fixed work: C = T + seg_cost x (non-empty
// sequences).  Workgroup b serves kv head g = b mod H_kv and takes the
// contiguous range [k C / N_g, (k+1) C / N_g) of that list, k = b / H_kv:
// every workgroup gets the same amount of work whatever the mix of lengths,
// and one whose range holds many short sequences gets fewer blocks for the
// segments it has to set up.  Within its range it walks segment by segment
// (one per sequence touched): a segment that is a whole sequence writes its
// output rows; a piece of a split sequence writes a partial, and the
// workgroup holding the sequence's first block records (first workgroup,
// number of pieces) for the merge kernel.
// Minimum waves per SIMD the compiler must leave room for: 3 for bf16 (about
// 154 VGPRs at head_dim 128, no spills); fp32 keeps its natural allocation.
// The VALU variant holds 8 dims x 8 heads of fp32 accumulators per lane and
// fits in 2 without spills.
template <bool BF16>
constexpr int kDecodeMinWaves = BF16 ? (PKV_DECODE_VALU_DOT ? 2 : 3) : 1;

template <bool BF16, int D, int BS, bool SH>
__global__ __launch_bounds__(kThreads, kDecodeMinWaves<BF16>) void decode_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<BF16, D> sm;
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  // Workgroup b = k * Hkv + g serves piece k of kv head g.  The hardware
  // deals consecutive workgroup ids round robin to the 8 XCDs, so with 8 kv
  // heads each XCD serves one head.  With shared blocks that is kept: a
  // head's shared blocks are then fetched into one L2 and found there by
  // its other sequences (400 forked samples: 285 against 542 us with the
  // heads spread).  Without sharing, at block size 16, the ids are dealt so
  // that each XCD runs a contiguous run of b, i.e. every head's pieces
  // (0.6-1 % faster on the 32k layer and the 8B-shaped batch); at block
  // size 32 one head per XCD measured 1 % faster and is kept.
  const int n_wg = static_cast<int>(gridDim.x);
  const int b = (!SH && BS == 16 && n_wg % 8 == 0)
                    ? static_cast<int>(blockIdx.x % 8) * (n_wg / 8) + static_cast<int>(blockIdx.x / 8)
                    : static_cast<int>(blockIdx.x);
  const int g = b % Hkv;
  const int k = b / Hkv;
  const bool appending = a.k_new != nullptr;
  if (threadIdx.x == 0) {
    sm.append_src[0] = a.k_new;
    sm.append_src[1] = a.v_new;
  }  // ordered before the reads by the barriers of the length scans

  // Cost of the head's list: each non-empty sequence counts its blocks plus
  // seg_cost, the fixed work of one segment (block ids, query, first loads,
  // cross-wave merge) in block units.
  auto cost_of = [&](int nb) { return nb > 0 ? nb + a.seg_cost : 0; };
  auto blocks_of = [&](int Lr) { return (clamp_len(Lr, a.max_context_len) + BS - 1) / BS; };
  // Sequence s holds [pre, pre + cost) of the list: the charge first, then
  // its blocks at [pre + seg_cost, pre + cost).  The first sequence touched
  // is the one whose interval holds c0.
  const bool small = S <= kThreads;
  int C = 0, s = 0, pre = 0;
  int64_t c0 = 0, c1 = 0;
  if (small) {
    // One scan: each thread keeps its sequence's inclusive prefix, and the
    // lengths stay in LDS for the walk.
    const int sq = threadIdx.x;
    int cst = 0;
    if (sq < S) {
      const int Lr = a.context_lens[sq];
      if ((Lr < 0 || Lr > a.max_context_len) && k == 0) report(a.status, PKV_DEV_BAD_LENGTH);
      sm.lens[sq] = Lr;
      cst = cost_of(blocks_of(Lr));
    }
    if (threadIdx.x == 0) sm.found_seq = -1;
    const int incl = block_scan<BF16, D>(cst, &C, sm);
    const int Ng = a.wgs_per_head < C ? a.wgs_per_head : C;
    if (k >= Ng) return;  // workgroup-uniform
    c0 = static_cast<int64_t>(k) * C / Ng;
    c1 = static_cast<int64_t>(k + 1) * C / Ng;
    if (cst > 0 && incl > c0 && incl - cst <= c0) {
      sm.found_seq = sq;
      sm.found_pre = incl - cst;
    }
    __syncthreads();
    s = sm.found_seq;  // found: c0 < C lies in one sequence's interval
    pre = sm.found_pre;
  } else {
    for (int base = 0; base < S; base += kThreads) {
      const int sq = base + threadIdx.x;
      int cst = 0;
      if (sq < S) {
        const int Lr = a.context_lens[sq];
        if ((Lr < 0 || Lr > a.max_context_len) && k == 0) report(a.status, PKV_DEV_BAD_LENGTH);
        cst = cost_of(blocks_of(Lr));
      }
      int tot;
      block_scan<BF16, D>(cst, &tot, sm);
      C += tot;
    }
    const int Ng = a.wgs_per_head < C ? a.wgs_per_head : C;
    if (k >= Ng) return;
    c0 = static_cast<int64_t>(k) * C / Ng;
    c1 = static_cast<int64_t>(k + 1) * C / Ng;
    int run = 0;
    for (int base = 0; base < S; base += kThreads) {
      if (threadIdx.x == 0) sm.found_seq = -1;
      const int sq = base + threadIdx.x;
      const int cst = sq < S ? cost_of(blocks_of(a.context_lens[sq])) : 0;
      int tot;
      const int incl = run + block_scan<BF16, D>(cst, &tot, sm);
      if (sq < S && cst > 0 && incl > c0 && incl - cst <= c0) {
        sm.found_seq = sq;
        sm.found_pre = incl - cst;
      }
      __syncthreads();
      const int fs = sm.found_seq;
      const int fp = sm.found_pre;
      __syncthreads();
      if (fs >= 0) {
        s = fs;
        pre = fp;
        break;
      }
      run += tot;
    }
  }
  const int Ng = a.wgs_per_head < C ? a.wgs_per_head : C;

  // Walk the segments: the sequences whose blocks meet [c0, c1).  Every one
  // visited holds at least one block of the range (lb0 < lb1).
  for (; s < S && static_cast<int64_t>(pre) + a.seg_cost < c1; ++s) {
    const int Lr = small ? __builtin_amdgcn_readfirstlane(sm.lens[s]) : a.context_lens[s];
    const int L = clamp_len(Lr, a.max_context_len);
    const int nb = (L + BS - 1) / BS;
    if (nb == 0) continue;
    const int64_t x0 = static_cast<int64_t>(pre) + a.seg_cost;  // list position of block 0
    const int lb0 = static_cast<int>((c0 > x0 ? c0 : x0) - x0);
    const int lb1 = static_cast<int>((c1 < x0 + nb ? c1 : x0 + nb) - x0);
    const bool whole = lb0 == 0 && lb1 == nb;
    const int prow = whole ? -1 : (b * 2 + (lb0 == 0 ? 1 : 0));
    // A length outside [1, max_context_len] appends nothing: a clamped length
    // would name a slot that already holds a cached token.
    const bool app = appending && lb1 == nb && Lr == L;
#if PKV_DECODE_VALU_DOT
    if constexpr (BF16) {
      if (a.group <= 4)
        decode_segment_valu<D, BS, 4, SH>(a, s, g, L, lb0, lb1, prow, app, sm);
      else
        decode_segment_valu<D, BS, 8, SH>(a, s, g, L, lb0, lb1, prow, app, sm);
    } else
#endif
      decode_segment<BF16, D, BS, SH>(a, s, g, L, lb0, lb1, prow, app, sm);
    if (lb0 == 0 && threadIdx.x == 0) {
      // Workgroup (within this head) whose range holds list position x: the
      // largest k' with k' C / Ng <= x.
      const int64_t last = x0 + nb - 1;
      const int k_last = static_cast<int>(((last + 1) * Ng - 1) / C);
      int32_t* mt = a.meta + (static_cast<size_t>(s) * Hkv + g) * 2;
      mt[0] = k;
      mt[1] = k_last - k + 1;
    }
    pre += nb + a.seg_cost;
  }
}

// Log-sum-exp merge of the pieces of split sequences, and zero rows for
// empty ones.  One workgroup per (kv head, sequence); runs as its own
// launch, so every partial written by the decode kernel is visible.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
  const int g = blockIdx.x;
  const int s = blockIdx.y;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const size_t head0 = static_cast<size_t>(s) * a.num_q_heads + static_cast<size_t>(g) * G;
  // The length and the piece record are independent loads, issued together
  // (the record is stale, and unused, for an empty sequence).
  const int32_t* mt = a.meta + (static_cast<size_t>(s) * Hkv + g) * 2;
  const int Lraw = a.context_lens[s];
  const int first = mt[0];
  const int npieces = mt[1];
  const int L = clamp_len(Lraw, a.max_context_len);
  if (L == 0) {
    for (int e = threadIdx.x; e < G * D; e += kThreads) {
      if constexpr (BF16)
        static_cast<uint16_t*>(a.out)[head0 * D + e] = 0;
      else
        static_cast<float*>(a.out)[head0 * D + e] = 0.f;
    }
    return;
  }
  if (npieces <= 1) return;
  // Partial row of piece j: workgroup (first + j) of head g; slot 1 for the
  // first piece (it starts at the sequence's first block), slot 0 after.
  auto prow = [&](int j) { return ((first + j) * Hkv + g) * 2 + (j == 0 ? 1 : 0); };

  // Each thread owns 4 consecutive dims of one head and merges the pieces
  // kMergeChunk at a time: all of a chunk's loads (max, sum, accumulator
  // slice) are issued before any is used, so a chunk costs one memory round
  // trip.  Across chunks the running (max, sum, accumulator) is rescaled as
  // in the online softmax.
  constexpr int kMergeChunk = 8;
  for (int e = threadIdx.x * 4; e < G * D; e += kThreads * 4) {
    const int h = e / D;
    const int d = e - h * D;
    float M = -INFINITY;
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < npieces; j0 += kMergeChunk) {
      float mj[kMergeChunk], lj[kMergeChunk];
      float4 vj[kMergeChunk];
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        const int j = j0 + u < npieces ? j0 + u : npieces - 1;
        const size_t r = static_cast<size_t>(prow(j)) * G + h;
        mj[u] = a.ws_m[r];
        lj[u] = a.ws_l[r];
        vj[u] = *reinterpret_cast<const float4*>(a.ws_acc + r * D + d);
      }
      float Mc = M;
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u)
        if (j0 + u < npieces) Mc = fmaxf(Mc, mj[u]);
      // Every piece holds at least one valid token, so Mc is finite.
      const float c = __builtin_amdgcn_exp2f(M - Mc);
      den *= c;
      acc.x *= c;
      acc.y *= c;
      acc.z *= c;
      acc.w *= c;
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        const float f = j0 + u < npieces ? __builtin_amdgcn_exp2f(mj[u] - Mc) : 0.f;
        den += f * lj[u];
        acc.x += f * vj[u].x;
        acc.y += f * vj[u].y;
        acc.z += f * vj[u].z;
        acc.w += f * vj[u].w;
      }
      M = Mc;
    }
    const float inv = 1.f / den;
    const size_t o = (head0 + h) * D + d;
    if constexpr (BF16) {
      const uint32_t lo = f32_to_bf16_bits(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.y * inv)) << 16);
      const uint32_t hi = f32_to_bf16_bits(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(acc.w * inv)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// Writes 16-byte chunk c of kv head h of one token's K/V row (rows of
// k_new/v_new are [num_kv_heads][head_dim]) into pool slot `slot`.
template <int EB>
__device__ __forceinline__ void write_row_chunk(const char* __restrict__ k_row, const char* __restrict__ v_row,
                                                char* __restrict__ k_cache, char* __restrict__ v_cache, int64_t slot,
                                                int h, int c, int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size) {
  constexpr int X = 16 / EB;
  const int64_t b = slot / block_size;
  const int o = static_cast<int>(slot - b * block_size);
  const int64_t src = (static_cast<int64_t>(h) * head_dim + static_cast<int64_t>(c) * X) * EB;
  const uint4 kv = *reinterpret_cast<const uint4*>(k_row + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(v_row + src);
  const int64_t tile = (b * num_kv_heads + h) * static_cast<int64_t>(head_dim) * block_size;
  *reinterpret_cast<uint4*>(k_cache + ((tile + (static_cast<int64_t>(c) * block_size + o) * X) * EB)) = kv;
  const int64_t vdst = tile + static_cast<int64_t>(c) * X * block_size + o;
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
  if constexpr (EB == 2) {
    uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache);
#pragma unroll
    for (int i = 0; i < 8; ++i) vc[vdst + static_cast<int64_t>(i) * block_size] = static_cast<uint16_t>(w[i / 2] >> (16 * (i & 1)));
  } else {
    uint32_t* vc = reinterpret_cast<uint32_t*>(v_cache);
#pragma unroll
    for (int i = 0; i < 4; ++i) vc[vdst + static_cast<int64_t>(i) * block_size] = w[i];
  }
}

// Cache append: one thread per (token, kv head, 16-byte chunk of head_dim).
template <int EB>
__global__ __launch_bounds__(256) void append_kernel(const char* __restrict__ k_new, const char* __restrict__ v_new,
                                                     char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                     const int32_t* __restrict__ slot_mapping, int64_t total,
                                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                     int32_t num_blocks, int32_t* __restrict__ status) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int nch = head_dim / (16 / EB);
  const int c = static_cast<int>(idx % nch);
  const int64_t th = idx / nch;
  const int h = static_cast<int>(th % num_kv_heads);
  const int64_t t = th / num_kv_heads;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  if (static_cast<int64_t>(slot) >= static_cast<int64_t>(num_blocks) * block_size) {
    report(status, PKV_DEV_BAD_SLOT);
    return;
  }
  const int64_t row = t * num_kv_heads * head_dim * EB;
  write_row_chunk<EB>(k_new + row, v_new + row, k_cache, v_cache, slot, h, c, num_kv_heads, head_dim, block_size);
}

// The decode step's one-token append as its own launch: sequence s's row
// goes to the slot of position L - 1 (L = its context length), found
// through its block table.  L == 0 skips it; a length outside
// [0, max_context_len] or a block id outside the pool skips it and is
// reported.  One thread per (sequence, kv head, 16-byte chunk).
template <int EB>
__global__ __launch_bounds__(256) void append_last_kernel(const char* __restrict__ k_new,
                                                          const char* __restrict__ v_new, char* __restrict__ k_cache,
                                                          char* __restrict__ v_cache,
                                                          const int32_t* __restrict__ block_tables,
                                                          const int32_t* __restrict__ context_lens, int64_t total,
                                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                          int32_t num_blocks, int32_t max_blocks_per_seq,
                                                          int32_t max_context_len, int32_t* __restrict__ status) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int nch = head_dim / (16 / EB);
  const int c = static_cast<int>(idx % nch);
  const int64_t th = idx / nch;
  const int h = static_cast<int>(th % num_kv_heads);
  const int64_t s = th / num_kv_heads;
  const int L = context_lens[s];
  if (L == 0) return;
  if (L < 0 || L > max_context_len) {
    if (c == 0 && h == 0) report(status, PKV_DEV_BAD_LENGTH);
    return;
  }
  const int32_t blk = block_tables[s * max_blocks_per_seq + (L - 1) / block_size];
  if (blk < 0 || blk >= num_blocks) {
    if (c == 0 && h == 0) report(status, PKV_DEV_BAD_BLOCK_ID);
    return;
  }
  const int64_t slot = static_cast<int64_t>(blk) * block_size + (L - 1) % block_size;
  const int64_t row = s * num_kv_heads * head_dim * EB;
  write_row_chunk<EB>(k_new + row, v_new + row, k_cache, v_cache, slot, h, c, num_kv_heads, head_dim, block_size);
}

// Block copy: blockIdx.x = pair, blockIdx.y = 0 (K pool) or 1 (V pool).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                          const int32_t* __restrict__ src_dst, int64_t block_bytes,
                                                          int32_t num_blocks, int32_t* __restrict__ status) {
  const int pair = blockIdx.x;
  const int32_t src = src_dst[2 * pair];
  const int32_t dst = src_dst[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    if (threadIdx.x == 0 && blockIdx.y == 0) report(status, PKV_DEV_BAD_PAIR);
    return;
  }
  char* pool = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* from = reinterpret_cast<const uint4*>(pool + static_cast<int64_t>(src) * block_bytes);
  uint4* to = reinterpret_cast<uint4*>(pool + static_cast<int64_t>(dst) * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) to[i] = from[i];
}

// Decode-step staging: copies the record written by pkv_bm_stage_step from
// pinned host memory (read in place over the bus) into the device buffers:
// slots, lengths, copy-on-write pairs, and the changed block-table entries.
__global__ __launch_bounds__(256) void stage_kernel(const int32_t* __restrict__ stage, int32_t n, int32_t np,
                                                   int32_t nu, int32_t width, int32_t* __restrict__ slots,
                                                   int32_t* __restrict__ lens, int32_t* __restrict__ pairs,
                                                   int32_t* __restrict__ tables, int32_t* __restrict__ status) {
  const int32_t* s_slots = stage + 4;
  const int32_t* s_lens = s_slots + n;
  const int32_t* s_pairs = s_lens + n;
  const int32_t* s_upd = s_pairs + 2 * np;
  const int64_t total = 2LL * n + 2LL * np + nu;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (i < n) {
      slots[i] = s_slots[i];
    } else if (i < 2LL * n) {
      lens[i - n] = s_lens[i - n];
    } else if (i < 2LL * n + 2LL * np) {
      pairs[i - 2LL * n] = s_pairs[i - 2LL * n];
    } else {
      const int64_t u = i - 2LL * n - 2LL * np;
      const int32_t row = s_upd[3 * u];
      const int32_t col = s_upd[3 * u + 1];
      if (row >= 0 && row < n && col >= 0 && col < width)
        tables[static_cast<int64_t>(row) * width + col] = s_upd[3 * u + 2];
      else
        report(status, PKV_DEV_BAD_RECORD);
    }
  }
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

// Workgroups per kv head.  partition_size == 0: one round of resident
// workgroups (compute units x occupancy, at most kMaxOcc per unit) spread
// over the kv heads; partition_size > 0: about partition_size tokens per
// workgroup for a batch of num_seqs x max_context_len tokens.
constexpr int kMaxOcc = 8;
constexpr int64_t kMaxWgsPerHead = 1 << 20;

int64_t wgs_per_head_for(int64_t num_seqs, int64_t num_kv_heads, int64_t max_context_len, int32_t partition_size,
                         int64_t cus, int64_t occ) {
  int64_t n;
  if (partition_size == 0) {
    const int64_t slots = cus * (occ < kMaxOcc ? occ : kMaxOcc);
    n = slots / num_kv_heads;
  } else {
    n = (num_seqs * max_context_len + partition_size - 1) / partition_size;
  }
  if (n < 1) n = 1;
  if (n > kMaxWgsPerHead) n = kMaxWgsPerHead;
  return n;
}

// Fixed work of one decode segment (block-id staging, query load, the first
// K/V round trip, the cross-wave merge and its output or partial), as a
// number of blocks of K/V streaming that take as long; the balanced split
// charges it per sequence.
constexpr int kSegmentCostTokens = 128;

int32_t segment_cost_blocks(int32_t block_size) {
  return static_cast<int32_t>((kSegmentCostTokens + block_size - 1) / block_size);
}

// Workspace: 256-byte aligned regions
//   meta int32[S*Hkv*2] | m float[N*2*G] | l float[N*2*G] | acc float[N*2*G*D]
struct WsLayout {
  int64_t meta, m, l, acc, total;
};

inline int64_t align256(int64_t x) { return ((x + 255) / 256) * 256; }

WsLayout ws_layout(int64_t num_seqs, int64_t num_kv_heads, int64_t group, int64_t head_dim, int64_t nwg) {
  WsLayout w;
  const int64_t rows = nwg * 2 * group;
  w.meta = 0;
  w.m = w.meta + align256(4 * num_seqs * num_kv_heads * 2);
  w.l = w.m + align256(4 * rows);
  w.acc = w.l + align256(4 * rows);
  w.total = w.acc + align256(4 * rows * head_dim);
  return w;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Resident workgroups per compute unit of one decode instantiation (cached).
template <bool BF16, int D, int BS>
int decode_occupancy() {
  static std::atomic<int> occ{0};
  int v = occ.load(std::memory_order_relaxed);
  if (v > 0) return v;
  // the smaller of the two cache-policy variants' (equal in practice), so
  // the grid and the workspace size do not depend on the call's flags
  int n0 = 0, n1 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n0, decode_kernel<BF16, D, BS, false>, kThreads, 0) != hipSuccess)
    n0 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n1, decode_kernel<BF16, D, BS, true>, kThreads, 0) != hipSuccess)
    n1 = 0;
  int n = n0 < n1 ? n0 : n1;
  if (n <= 0) n = 1;
  occ.store(n, std::memory_order_relaxed);
  return n;
}

int occupancy_for(pkv_dtype dt, int32_t head_dim, int32_t block_size) {
  if (dt == PKV_BF16) {
    if (head_dim == 128) return block_size == 16 ? decode_occupancy<true, 128, 16>() : decode_occupancy<true, 128, 32>();
    return block_size == 16 ? decode_occupancy<true, 64, 16>() : decode_occupancy<true, 64, 32>();
  }
  if (head_dim == 128) return block_size == 16 ? decode_occupancy<false, 128, 16>() : decode_occupancy<false, 128, 32>();
  return block_size == 16 ? decode_occupancy<false, 64, 16>() : decode_occupancy<false, 64, 32>();
}

template <bool BF16, int D, int BS>
void launch_decode(const DecodeArgs& a, bool shared, hipStream_t st) {
  const uint32_t nwg = static_cast<uint32_t>(static_cast<int64_t>(a.wgs_per_head) * a.num_kv_heads);
  if (shared)
    decode_kernel<BF16, D, BS, true><<<dim3(nwg), kThreads, 0, st>>>(a);
  else
    decode_kernel<BF16, D, BS, false><<<dim3(nwg), kThreads, 0, st>>>(a);
  decode_merge_kernel<BF16, D><<<dim3(a.num_kv_heads, a.num_seqs), kThreads, 0, st>>>(a);
}

template <bool BF16, int D>
void dispatch_bs(const DecodeArgs& a, int32_t bs, bool shared, hipStream_t st) {
  if (bs == 16)
    launch_decode<BF16, D, 16>(a, shared, st);
  else
    launch_decode<BF16, D, 32>(a, shared, st);
}

}  // namespace

// The device status word: every GPU the library runs on holds its own copy
// (kernels reach it through the address pkv::device_status_ptr returns for
// the current device).
__device__ int32_t g_pkv_device_status;

namespace pkv {
std::string& last_error_slot() {
  thread_local std::string msg;
  return msg;
}

int32_t stage_device_ptr(const int32_t* stage, const int32_t** dev_out) {
  // Looked up on every call (nothing is cached): a pinned buffer may be
  // freed and its address reused by pageable memory, which the GPU cannot
  // read.  Both queries are host-side table lookups, microseconds against
  // a decode step.
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, stage) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(PKV_ERR_INVALID_ARG, "stage buffer is not pinned host memory (hipHostMalloc / pin_memory)");
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<int32_t*>(stage), 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return fail(PKV_ERR_INVALID_ARG, "stage buffer is not pinned host memory (hipHostMalloc / pin_memory)");
  }
  *dev_out = static_cast<const int32_t*>(d);
  return PKV_OK;
}

int32_t device_status_ptr(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(PKV_ERR_DEVICE, "no usable current device for the status word");
  }
  int32_t* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_pkv_device_status));
    if (e != hipSuccess || !addr) {
      (void)hipGetLastError();
      return fail(PKV_ERR_DEVICE, "status word address: %s", hipGetErrorString(e));
    }
    p = static_cast<int32_t*>(addr);
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

int32_t launch_stage(const int32_t* stage_dev, int32_t n_seqs, int32_t n_pairs, int32_t n_updates, int32_t width,
                     int32_t* slot_mapping, int32_t* context_lens, int32_t* cow_pairs, int32_t* block_tables,
                     void* stream) {
  int32_t* status = nullptr;
  if (int32_t e = device_status_ptr(&status)) return e;
  const int64_t total = 2LL * n_seqs + 2LL * n_pairs + n_updates;
  int64_t grid = (total + 255) / 256;
  if (grid > 1024) grid = 1024;
  if (grid < 1) grid = 1;
  stage_kernel<<<dim3(static_cast<uint32_t>(grid)), 256, 0, static_cast<hipStream_t>(stream)>>>(
      stage_dev, n_seqs, n_pairs, n_updates, width, slot_mapping, context_lens, cow_pairs, block_tables, status);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, "stage launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return pkv::last_error_slot().c_str(); }

int32_t pkv_version(void) { return 101; }

int32_t pkv_device_status(void* stream, int32_t clear, int32_t* flags_out) {
  if (!flags_out) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  int32_t* status = nullptr;
  if (int32_t e = pkv::device_status_ptr(&status)) return e;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  int32_t v = 0;
  if (e == hipSuccess) e = hipMemcpy(&v, status, sizeof(v), hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const int32_t zero = 0;
    e = hipMemcpy(status, &zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return pkv::fail(PKV_ERR_DEVICE, "reading the device status word: %s", hipGetErrorString(e));
  }
  *flags_out = v;
  return pkv::ok();
}

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
  int32_t* status = nullptr;
  if (int32_t e = pkv::device_status_ptr(&status)) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (eb == 2)
    append_kernel<2><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, st>>>(
        static_cast<const char*>(k_new), static_cast<const char*>(v_new), static_cast<char*>(k_cache),
        static_cast<char*>(v_cache), slot_mapping, total, num_kv_heads, head_dim, block_size, num_blocks, status);
  else
    append_kernel<4><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, st>>>(
        static_cast<const char*>(k_new), static_cast<const char*>(v_new), static_cast<char*>(k_cache),
        static_cast<char*>(v_cache), slot_mapping, total, num_kv_heads, head_dim, block_size, num_blocks, status);
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
  int32_t* status = nullptr;
  if (int32_t e = pkv::device_status_ptr(&status)) return e;
  copy_blocks_kernel<<<dim3(num_pairs, 2), 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<char*>(k_cache), static_cast<char*>(v_cache), src_dst, block_bytes, num_blocks, status);
  return launch_status("paged_kv_copy_blocks");
}

int32_t paged_attention_workgroups_per_head(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_context_len, int32_t partition_size,
                                            pkv_dtype dt) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0 || partition_size < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes");
  const int64_t n = wgs_per_head_for(num_seqs, num_kv_heads, max_context_len, partition_size, device_cus(),
                                     occupancy_for(dt, head_dim, block_size));
  pkv::ok();
  return static_cast<int32_t>(n);
}

int32_t paged_attention_segment_cost(int32_t block_size) {
  if (block_size != 16 && block_size != 32) return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported", block_size);
  pkv::ok();
  return segment_cost_blocks(block_size);
}

size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_context_len, int32_t partition_size) {
  if (check_common(head_dim, block_size, PKV_BF16)) return 0;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 || partition_size < 0 ||
      num_q_heads % num_kv_heads) {
    pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes");
    return 0;
  }
  pkv::ok();
  if (num_seqs == 0) return 0;
  // Sized for the largest occupancy the launch may use, so the size does not
  // depend on the element type.
  const int64_t n = wgs_per_head_for(num_seqs, num_kv_heads, max_context_len, partition_size, device_cus(), kMaxOcc);
  return static_cast<size_t>(ws_layout(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                       n * num_kv_heads).total);
}

}  // extern "C"

namespace {

// Both decode entry points: validation, workspace layout and launch.
// k_new/v_new null: decode only; else the token at position L - 1 of each
// sequence is appended from them first.
int32_t decode_call(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dt, uint32_t flags,
                    void* stream, const char* what) {
  if (int32_t e = check_common(head_dim, block_size, dt)) return e;
  if (flags & ~static_cast<uint32_t>(PKV_DECODE_SHARED_BLOCKS))
    return pkv::fail(PKV_ERR_INVALID_ARG, "unknown decode flags 0x%x", flags);
  const bool shared = (flags & PKV_DECODE_SHARED_BLOCKS) != 0;
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
  if (!aligned16(k_new) || !aligned16(v_new))
    return pkv::fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  if (partition_size < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "partition_size %d < 0", partition_size);
  if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs * max_blocks_per_seq exceeds the int32 range");
  const int64_t wph = wgs_per_head_for(num_seqs, num_kv_heads, max_context_len, partition_size, device_cus(),
                                       occupancy_for(dt, head_dim, block_size));
  if (wph * num_kv_heads > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "too many workgroups");
  const WsLayout wl = ws_layout(num_seqs, num_kv_heads, G, head_dim, wph * num_kv_heads);
  const size_t need = static_cast<size_t>(wl.total);
  if (!workspace || workspace_bytes < need)
    return pkv::fail(PKV_ERR_CAPACITY, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int32_t* status = nullptr;
  if (int32_t e = pkv::device_status_ptr(&status)) return e;
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  // The append is folded into the decode kernel only when there are at
  // most as many sequences as decode workgroups per kv head, so there is on
  // average at most one appended (sequence, kv head) row per workgroup (a
  // workgroup whose range holds several short sequences still writes one row
  // for each).  Each row's V part is head_dim two-byte stores (the V tile
  // is dimension-major); many of them issued into the decode kernel's
  // saturated read stream cost more than a separate launch (measured: +27 us
  // on 256 sequences x 8 kv heads over 768 workgroups, against -4 us of
  // launch saved on 16 x 8).  Both ways write the same bytes.
  const bool fold = k_new != nullptr && static_cast<int64_t>(num_seqs) <= wph;
  if (k_new != nullptr && !fold) {
    const int eb = dt == PKV_BF16 ? 2 : 4;
    const int64_t total = static_cast<int64_t>(num_seqs) * num_kv_heads * (head_dim * eb / 16);
    const int64_t blocks = (total + 255) / 256;
    hipStream_t ast = static_cast<hipStream_t>(stream);
    if (eb == 2)
      append_last_kernel<2><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, ast>>>(
          static_cast<const char*>(k_new), static_cast<const char*>(v_new),
          const_cast<char*>(static_cast<const char*>(k_cache)), const_cast<char*>(static_cast<const char*>(v_cache)),
          block_tables, context_lens, total, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
          max_context_len, status);
    else
      append_last_kernel<4><<<dim3(static_cast<uint32_t>(blocks)), 256, 0, ast>>>(
          static_cast<const char*>(k_new), static_cast<const char*>(v_new),
          const_cast<char*>(static_cast<const char*>(k_cache)), const_cast<char*>(static_cast<const char*>(v_cache)),
          block_tables, context_lens, total, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
          max_context_len, status);
  }
  a.k_new = fold ? k_new : nullptr;
  a.v_new = fold ? v_new : nullptr;
  char* ws = static_cast<char*>(workspace);
  a.meta = reinterpret_cast<int32_t*>(ws + wl.meta);
  a.ws_m = reinterpret_cast<float*>(ws + wl.m);
  a.ws_l = reinterpret_cast<float*>(ws + wl.l);
  a.ws_acc = reinterpret_cast<float*>(ws + wl.acc);
  a.status = status;
  a.wgs_per_head = static_cast<int32_t>(wph);
  a.seg_cost = segment_cost_blocks(block_size);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == PKV_BF16) {
    if (head_dim == 128)
      dispatch_bs<true, 128>(a, block_size, shared, st);
    else
      dispatch_bs<true, 64>(a, block_size, shared, st);
  } else {
    if (head_dim == 128)
      dispatch_bs<false, 128>(a, block_size, shared, st);
    else
      dispatch_bs<false, 64>(a, block_size, shared, st);
  }
  return launch_status(what);
}

// Scratch of the allocation-free decode call: the decode workspace (piece
// records and partials) of one call, held by every GPU the library runs on
// until the process ends.  Host code never names the array itself (its
// name is a host-side stand-in, not a device address); it uses the address
// scratch_ptr returns for the current device.
constexpr size_t kScratchBytes = size_t{32} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current GPU's scratch array, looked up once per
// device with that device current.
int32_t scratch_ptr(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return pkv::fail(PKV_ERR_DEVICE, "no usable current device for the decode scratch");
  }
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return pkv::fail(PKV_ERR_DEVICE, "decode scratch address: %s", hipGetErrorString(e));
    }
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dt,
                               uint32_t flags, void* stream) {
  return decode_call(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dt, flags, stream, "paged_attention_decode");
}

int32_t paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype dt, uint32_t flags, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  return decode_call(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dt, flags, stream, "paged_attention_decode_append");
}

int32_t paged_attention_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_cache, void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                              float scale, int32_t partition_size, pkv_dtype dt, uint32_t flags,
                                              void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_seqs <= 0)  // validation only; nothing to launch
    return decode_call(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       partition_size, nullptr, 0, dt, flags, stream, "paged_attention_decode_append_noalloc");
  void* ws = nullptr;
  if (int32_t e = scratch_ptr(&ws)) return e;
  // decode_call rejects a request whose workspace exceeds the scratch with
  // PKV_ERR_CAPACITY before launching anything.
  const int32_t st = decode_call(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs,
                                 num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                 max_context_len, scale, partition_size, ws, kScratchBytes, dt, flags, stream,
                                 "paged_attention_decode_append_noalloc");
  if (st == PKV_ERR_CAPACITY)
    pkv::fail(PKV_ERR_CAPACITY, "paged_attention_decode_append_noalloc: %s (the built-in scratch holds %zu bytes)",
              pkv_last_error(), kScratchBytes);
  return st;
}

}  // extern "C"
