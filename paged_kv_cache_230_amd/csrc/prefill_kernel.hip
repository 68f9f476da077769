// Chunked-prefill attention over the paged KV cache for gfx950 (MI355X).
//
// A chunk of each sequence's newest C tokens (their K/V already appended)
// attends causally over the sequence's cache: the token at position p reads
// positions 0..p.  This is the prefill phase whose K/V the cache then holds
// ("PagedAttention et RadixAttention : parlons de KV Cache", the part on the
// two independent problems, and the closing part on prefix caching, which
// skips the prefill of prefixes already seen); the cache is read through
// the block tables exactly as in decode (same page, PagedAttention section,
// step 2), and paging leaves the result unchanged (its closing paragraph).
//
// Kernel design (gfx950, wave64, bf16 matrix cores):
//   * One workgroup = 4 waves = one (query tile, kv head, sequence).  The
//     128 score rows of a tile are (query token, query head) pairs of the
//     G heads sharing the kv head, so every K/V byte staged serves G heads.
//     Wave w owns rows 32w..32w+31 as two 16-row sets.
//   * Keys advance 32 per step.  The step's K and V block tiles are copied
//     into LDS in the pool's own format (double-buffered: the next step's
//     global loads are in flight during this step's matrix work); block ids
//     come from uniform (scalar) loads.  V slots past the context are
//     zeroed in LDS, so unused slots of the last block never reach the
//     products.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: keys in the A operand (one
//     16-byte LDS read per lane serves both row sets), query rows in the
//     columns.  Lane l holds the scores of keys 4(l/16)+i (+16) of row l%16,
//     which is the B-operand layout of the PV product once its 32 keys are
//     ordered the same way in A: O^T += V^T P^T, again 16x16x32.
//   * Online softmax per row in the log2 domain; row maxima by gfx950 row
//     swaps (v_permlane16/32_swap), not LDS shuffles; the causal mask (a
//     select, never a multiply) only on the steps that reach past the tile's
//     first position.  A row's reference max moves only when its max grows
//     by more than 2^8, so the accumulators are rescaled rarely; the
//     probabilities then stay below 2^8, well inside fp32 and bf16 range.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pkv_status.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float float4v;

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRowSets = 2;                   // 16-row sets per wave
constexpr int kRows = kPWaves * kRowSets * 16;  // score rows per workgroup
constexpr int kKeys = 32;                     // keys per step

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t tokens_per_tile;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_query_len;
  float scale_log2;
};

// One step's K and V in LDS.  K part: [kKeys/BS tiles][D/8][BS][8] bf16,
// the pool's tile format (the QK A operand is then one contiguous 1 KiB run
// per wave).  V part: [D][4 lane groups][8] bf16, where group g holds keys
// 4g..4g+3 and 16+4g..16+4g+3 of the step, the order of the PV product's
// k index, so each A operand is one 16-byte read.
template <int D>
struct StageLayout {
  static constexpr int kBytes = kKeys * D * 2;  // K or V part
  static constexpr int kUint4 = 2 * kBytes / 16;
  static constexpr int kPerThread = kUint4 / kPThreads;
  static_assert(kUint4 % kPThreads == 0, "stage must split evenly over the threads");
};

template <int D>
struct PrefillSmem {
  uint4 stage[2][StageLayout<D>::kUint4];
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Combine the 4 lanes l, l^16, l^32, l^48 (the four 16-lane rows of a
// wave) with the gfx950 row swaps: v_permlane16_swap(x, y) exchanges the
// odd rows of x with the even rows of y, v_permlane32_swap the upper half
// of x with the lower half of y; with y = x, the two results hold every
// lane's own value and its partner's, in some order.  Each result passes
// through an empty asm statement before it is combined: the compiler in
// use otherwise reads the first result twice when one instruction consumes
// both (it turns max(r0, r1) into r0 and r0 + r1 into r0 + r0).
__device__ __forceinline__ float opaque_f(uint32_t v) {
  asm volatile("" : "+v"(v));
  return __builtin_bit_cast(float, v);
}

template <bool kMax>
__device__ __forceinline__ float reduce4rows(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float a0 = opaque_f(a[0]), a1 = opaque_f(a[1]);
  v = kMax ? fmaxf(a0, a1) : a0 + a1;
  u = __builtin_bit_cast(uint32_t, v);
  auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float b0 = opaque_f(b[0]), b1 = opaque_f(b[1]);
  return kMax ? fmaxf(b0, b1) : b0 + b1;
}

// Where each of a thread's 16-byte staging chunks comes from and goes to;
// the same every step, only the block ids change.
template <int D, int BS>
struct StagePlan {
  static constexpr int kTileBytes = BS * D * 2;
  int src[StageLayout<D>::kPerThread];   // byte offset inside the (block, kv head) tile
  int tile[StageLayout<D>::kPerThread];  // tile of the step (0 .. kKeys/BS-1)
  int dst[StageLayout<D>::kPerThread];   // K: byte offset in the K part; V: first key of the chunk in the step
  int dim[StageLayout<D>::kPerThread];   // V: the chunk's dim
  __device__ StagePlan() {
    // Chunk k of a thread lies in the K part exactly when k < kPerThread / 2
    // (the K part is the first half of the stage and threads stride it).
    constexpr int kHalf = StageLayout<D>::kPerThread / 2;
#pragma unroll
    for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
      const int ov = (threadIdx.x + kPThreads * (k % kHalf)) * 16;
      tile[k] = ov / kTileBytes;
      src[k] = ov % kTileBytes;
      dst[k] = k < kHalf ? ov : tile[k] * BS + (src[k] % (2 * BS)) / 2;  // V: first key of the chunk in the step
      dim[k] = k < kHalf ? 0 : src[k] / (2 * BS);                        // V tile [D][BS]: 8 keys of one dim
    }
  }
};

template <int D, int BS>
__device__ __forceinline__ void load_stage(const PrefillArgs& a, const StagePlan<D, BS>& pl, int g, int L,
                                           const int32_t* table, int st, uint4 (&r)[StageLayout<D>::kPerThread]) {
  constexpr int kTiles = kKeys / BS;
  int32_t ids[kTiles];
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) {
    const int lb = st * kTiles + kt;
    ids[kt] = lb * BS < L ? clampi(table[lb], 0, a.num_blocks - 1) : -1;
  }
#pragma unroll
  for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
    constexpr int kHalf = StageLayout<D>::kPerThread / 2;  // first half of the chunks is K
    int id = ids[0];
#pragma unroll
    for (int kt = 1; kt < kTiles; ++kt) id = pl.tile[k] == kt ? ids[kt] : id;  // select: no dynamic indexing
    const char* base = static_cast<const char*>(k < kHalf ? a.k_cache : a.v_cache);
    r[k] = id >= 0 ? *reinterpret_cast<const uint4*>(base + (static_cast<int64_t>(id) * a.num_kv_heads + g) *
                                                              StagePlan<D, BS>::kTileBytes + pl.src[k])
                   : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int BS>
__device__ __forceinline__ void store_stage(char* dst, const StagePlan<D, BS>& pl, int key_base, int L,
                                            uint4 (&r)[StageLayout<D>::kPerThread]) {
  constexpr int kHalf = StageLayout<D>::kPerThread / 2;
#pragma unroll
  for (int k = 0; k < kHalf; ++k) *reinterpret_cast<uint4*>(dst + pl.dst[k]) = r[k];
  char* vdst = dst + StageLayout<D>::kBytes;
  const bool tail = key_base + kKeys > L;  // uniform: only the step holding the context's end
#pragma unroll
  for (int k = kHalf; k < StageLayout<D>::kPerThread; ++k) {
    uint4 x = r[k];
    const int kk0 = pl.dst[k];  // first key of the chunk within the step (a multiple of 8)
    if (tail) {  // zero V slots at or past the context end
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key_base + kk0 + e >= L) w[e / 2] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      x = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const int half = kk0 / 16, g0 = (kk0 % 16) / 4;
    char* row = vdst + pl.dim[k] * 64 + half * 8;
    *reinterpret_cast<uint2*>(row + g0 * 16) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2*>(row + (g0 + 1) * 16) = make_uint2(x.z, x.w);
  }
}

template <int D, int BS>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillSmem<D> sm;
  constexpr int kTileBytes = BS * D * 2;
  constexpr int kChunks = D / 32;  // 32-dim slices of the QK contraction
  constexpr int kDimTiles = D / 16;
  // The reference max of a row moves only when the row max exceeds it by
  // more than this (log2 units), so probabilities stay below 2^8 and the
  // accumulators are rescaled only on such moves.
  constexpr float kSlack = 8.f;
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int L = clampi(a.context_lens[s], 0, a.max_blocks_per_seq * BS);
  int q0 = a.query_start[s];
  int C = a.query_start[s + 1] - q0;
  if (q0 < 0 || q0 > a.num_tokens) C = 0;
  C = clampi(C, 0, L < a.max_query_len ? L : a.max_query_len);
  if (q0 + C > a.num_tokens) C = a.num_tokens - q0;
  const int TQ = a.tokens_per_tile;
  const int ntiles = (C + TQ - 1) / TQ;
  const int tile = static_cast<int>(gridDim.x) - 1 - static_cast<int>(blockIdx.x);  // latest tiles first
  if (tile >= ntiles) return;
  const int tok0 = tile * TQ;
  const int ntok = C - tok0 < TQ ? C - tok0 : TQ;
  const int pos0 = L - C + tok0;  // position of the tile's first token
  const int kend = pos0 + ntok;   // keys [0, kend) are read
  const int nsteps = (kend + kKeys - 1) / kKeys;
  const int mask_from = (pos0 + 1) / kKeys;  // steps before this one see no key past pos0
  const int G = a.group;
  const int32_t* table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq;
  const StagePlan<D, BS> plan;

  // This lane's two rows (one per row set): token, head, position, validity.
  int row_pos[kRowSets];
  int64_t row_q[kRowSets];
  bool row_ok[kRowSets];
#pragma unroll
  for (int rs = 0; rs < kRowSets; ++rs) {
    const int r = wave * (kRowSets * 16) + rs * 16 + col;
    const int tq = r / G;
    const int j = r - tq * G;
    row_ok[rs] = tq < ntok;
    row_pos[rs] = row_ok[rs] ? pos0 + tq : kend - 1;
    row_q[rs] = row_ok[rs] ? (static_cast<int64_t>(q0 + tok0 + tq) * a.num_q_heads + g * G + j) * D : -1;
  }

  // Queries: B operand of the QK product, lane holds dims 8*grp..+8 of each 32-dim chunk.
  bf16x8 qb[kRowSets][kChunks];
#pragma unroll
  for (int rs = 0; rs < kRowSets; ++rs)
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row_ok[rs]) x = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.q) + row_q[rs] + c * 32 + grp * 8);
      qb[rs][c] = __builtin_bit_cast(bf16x8, x);
    }

  float4v acc[kRowSets][kDimTiles];
  float m_run[kRowSets], l_run[kRowSets];
#pragma unroll
  for (int rs = 0; rs < kRowSets; ++rs) {
    m_run[rs] = -INFINITY;
    l_run[rs] = 0.f;
#pragma unroll
    for (int t = 0; t < kDimTiles; ++t) acc[rs][t] = float4v{0.f, 0.f, 0.f, 0.f};
  }

  uint4 nxt[StageLayout<D>::kPerThread];
  load_stage<D, BS>(a, plan, g, L, table, 0, nxt);
  store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[0]), plan, 0, L, nxt);
  __syncthreads();

  for (int st = 0; st < nsteps; ++st) {
    const bool more = st + 1 < nsteps;
    if (more) load_stage<D, BS>(a, plan, g, L, table, st + 1, nxt);
    const char* kl = reinterpret_cast<const char*>(sm.stage[st & 1]);
    const char* vl = kl + StageLayout<D>::kBytes;

    // ---- S^T = K Q^T: two 16-key halves x two row sets.
    float4v sc[kRowSets][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = h * 16 + col;  // key within the step for the A operand
      const int kt = kk / BS, kb = kk % BS;
#pragma unroll
      for (int rs = 0; rs < kRowSets; ++rs) sc[rs][h] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + kt * kTileBytes + ((c * 4 + grp) * BS + kb) * 16);
#pragma unroll
        for (int rs = 0; rs < kRowSets; ++rs)
          sc[rs][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[rs][c], sc[rs][h], 0, 0, 0);
      }
    }

    // ---- online softmax per row; P packed as the B operand of the PV product.
    const bool masked = st >= mask_from;
    bf16x8 pb[kRowSets];
    float alpha[kRowSets];
    bool moved = false;
#pragma unroll
    for (int rs = 0; rs < kRowSets; ++rs) {
      float x[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[h * 4 + i] = sc[rs][h][i];
      if (masked) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (st * kKeys + h * 16 + grp * 4 + i > row_pos[rs]) x[h * 4 + i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = reduce4rows<true>(mx) * a.scale_log2;
      const bool move = mx > m_run[rs] + kSlack;
      const float m_use = move ? mx : m_run[rs];
      alpha[rs] = __builtin_amdgcn_exp2f(m_run[rs] - m_use);
      moved |= move;
      m_run[rs] = m_use;
      float sum = 0.f;
      __bf16 pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(x[e], a.scale_log2, -m_use));
        sum += p;
        pe[e] = static_cast<__bf16>(p);
      }
      l_run[rs] = l_run[rs] * alpha[rs] + sum;
      pb[rs] = bf16x8{pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]};
    }
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int rs = 0; rs < kRowSets; ++rs)
#pragma unroll
        for (int t = 0; t < kDimTiles; ++t) acc[rs][t] *= alpha[rs];
    }

    // ---- O^T += V^T P^T: A = V^T rows dim 16t+col, k index 8*grp+e = the
    // keys of lane group grp in the interleaved V layout.
#pragma unroll
    for (int t = 0; t < kDimTiles; ++t) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(vl + (t * 16 + col) * 64 + grp * 16);
#pragma unroll
      for (int rs = 0; rs < kRowSets; ++rs)
        acc[rs][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rs], acc[rs][t], 0, 0, 0);
    }

    if (more) store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[(st + 1) & 1]), plan, (st + 1) * kKeys, L, nxt);
    __syncthreads();
  }

  // ---- normalise and store: lane holds dims 16t + 4*grp + i of row col.
#pragma unroll
  for (int rs = 0; rs < kRowSets; ++rs) {
    const float l = reduce4rows<false>(l_run[rs]);
    if (!row_ok[rs]) continue;
    const float inv = 1.f / l;
    __bf16* orow = static_cast<__bf16*>(a.out) + row_q[rs];
#pragma unroll
    for (int t = 0; t < kDimTiles; ++t) {
      const __bf16 o0 = static_cast<__bf16>(acc[rs][t][0] * inv), o1 = static_cast<__bf16>(acc[rs][t][1] * inv);
      const __bf16 o2 = static_cast<__bf16>(acc[rs][t][2] * inv), o3 = static_cast<__bf16>(acc[rs][t][3] * inv);
      uint2 w;
      w.x = __builtin_bit_cast(uint16_t, o0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o1)) << 16);
      w.y = __builtin_bit_cast(uint16_t, o2) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o3)) << 16);
      *reinterpret_cast<uint2*>(orow + t * 16 + grp * 4) = w;
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int D>
void dispatch_prefill_bs(const PrefillArgs& a, int bs, dim3 grid, hipStream_t st) {
  if (bs == 16)
    prefill_kernel<D, 16><<<grid, kPThreads, 0, st>>>(a);
  else
    prefill_kernel<D, 32><<<grid, kPThreads, 0, st>>>(a);
}

}  // namespace

extern "C" {

int32_t paged_attention_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_query_len, float scale, pkv_dtype dt, void* stream) {
  if (dt != PKV_BF16) return pkv::fail(PKV_ERR_UNSUPPORTED, "paged_attention_prefill supports bf16 only");
  if (head_dim != 64 && head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported (16 or 32)", block_size);
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_query_len < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "bad sizes: num_seqs %d num_tokens %d num_q_heads %d num_kv_heads %d num_blocks %d "
                     "max_blocks_per_seq %d max_query_len %d",
                     num_seqs, num_tokens, num_q_heads, num_kv_heads, num_blocks, max_blocks_per_seq, max_query_len);
  if (num_q_heads % num_kv_heads)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                     num_kv_heads);
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > kRows) return pkv::fail(PKV_ERR_UNSUPPORTED, "query group size %d > %d not supported", G, kRows);
  if (num_seqs > 65535 || num_kv_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_seqs and num_kv_heads must be <= 65535");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX ||
      static_cast<int64_t>(num_seqs) * max_blocks_per_seq > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "table size exceeds the int32 range");
  if (!std::isfinite(scale) || !(scale > 0.f)) return pkv::fail(PKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (num_seqs == 0 || max_query_len == 0 || num_tokens == 0) return pkv::ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID_ARG, "q, out and the pools must be 16-byte aligned");
  const int32_t tq = kRows / G;
  const int64_t ntiles = (static_cast<int64_t>(max_query_len) + tq - 1) / tq;
  if (ntiles > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "max_query_len too large");
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.tokens_per_tile = tq;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<uint32_t>(ntiles), static_cast<uint32_t>(num_kv_heads), static_cast<uint32_t>(num_seqs));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    dispatch_prefill_bs<128>(a, block_size, grid, st);
  else
    dispatch_prefill_bs<64>(a, block_size, grid, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_DEVICE, "paged_attention_prefill launch: %s", hipGetErrorString(e));
  return pkv::ok();
}

}  // extern "C"
