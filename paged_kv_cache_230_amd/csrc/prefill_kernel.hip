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
//     Wave w owns rows 32w..32w+31, one per lane pair (l, l+32).
//   * Keys advance 32 per step.  The step's K and V block tiles are copied
//     into LDS in the pool's own format (double-buffered: the next step's
//     global loads are in flight during this step's matrix work); block ids
//     come from uniform (scalar) loads.  V slots past the context are
//     zeroed in LDS, so unused slots of the last block never reach the
//     products.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the step's 32 keys in the
//     rows, the wave's 32 query rows in the columns.  Lane l holds 16
//     scores of row l%32 (keys 8(j/4)+4(l/32)+j%4), so a row's max needs one
//     partner lane.  Those scores, in that order, are the B operand of the
//     PV product once A (V^T, read from LDS) orders its k index the same
//     way: O^T += V^T P^T, again 32x32x16.
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
typedef __attribute__((ext_vector_type(16))) float float16v;

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRows = kPWaves * 32;  // score rows per workgroup (32 per wave)
constexpr int kKeys = 32;                     // keys per step
// Block ids of the tile's key range are staged in LDS this many at a time
// (a vector load of a table entry per step would stall its wave).
constexpr int kIdChunk = 1024;

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
// the pool's tile format (each 16-lane quarter of a QK A operand read is a
// contiguous 256-byte run).  V part: [D][4 groups][8] bf16, group 2m+h
// holding keys 16m+4h+{0..3} then 16m+8+4h+{0..3}: the k order of PV
// product m for lanes with l/32 = h, so each A operand is one 16-byte read;
// rows are padded from 64 to 80 bytes so the 16 dims a quarter-wave reads
// fall in distinct banks.
constexpr int kVRow = 80;  // bytes per dim row of the V part
template <int D>
struct StageLayout {
  static constexpr int kBytes = kKeys * D * 2;  // data bytes of the K or the V part
  static constexpr int kVBytes = D * kVRow;     // V part with padding
  static constexpr int kStageBytes = kBytes + kVBytes;
  static constexpr int kPerThread = 2 * kBytes / 16 / kPThreads;  // 16-byte chunks per thread
  static_assert((2 * kBytes / 16) % kPThreads == 0, "stage must split evenly over the threads");
};

template <int D>
struct PrefillSmem {
  uint4 stage[2][StageLayout<D>::kStageBytes / 16];
  int32_t ids[kIdChunk];
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Combine lanes l and l^32 (the two holders of a score row) with the
// gfx950 swap v_permlane32_swap(x, y), which exchanges the upper half of x
// with the lower half of y: with y = x its two results hold every lane's
// own value and its partner's, in some order.  Each result passes through an
// empty asm statement before they are combined: the compiler in use
// otherwise reads the first result twice when one instruction consumes both
// (max(r0, r1) becomes r0, r0 + r1 becomes r0 + r0).
__device__ __forceinline__ float opaque_f(uint32_t v) {
  asm volatile("" : "+v"(v));
  return __builtin_bit_cast(float, v);
}

template <bool kMax>
__device__ __forceinline__ float reduce_pair(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float b0 = opaque_f(b[0]), b1 = opaque_f(b[1]);
  return kMax ? fmaxf(b0, b1) : b0 + b1;
}

// Where each of a thread's 16-byte staging chunks comes from and goes to;
// the same every step, only the block ids change.
template <int D, int BS>
struct StagePlan {
  static constexpr int kTileBytes = BS * D * 2;
  const char* base[StageLayout<D>::kPerThread];  // pool + kv head tile + src (add id * stride)
  int src[StageLayout<D>::kPerThread];   // byte offset inside the (block, kv head) tile
  int tile[StageLayout<D>::kPerThread];  // tile of the step (0 .. kKeys/BS-1)
  int dst[StageLayout<D>::kPerThread];   // K: byte offset in the K part; V: first key of the chunk in the step
  int dim[StageLayout<D>::kPerThread];   // V: the chunk's dim
  __device__ StagePlan(const PrefillArgs& a, int g) {
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
      base[k] = static_cast<const char*>(k < kHalf ? a.k_cache : a.v_cache) + g * kTileBytes + src[k];
    }
  }
};

// Staged block ids [chunk_base, chunk_base + kIdChunk) of the sequence,
// clamped to the pool; -1 past the context.
__device__ __forceinline__ void fill_ids(const PrefillArgs& a, const int32_t* table, int chunk_base, int nblk,
                                         int32_t* ids) {
  for (int i = threadIdx.x; i < kIdChunk; i += kPThreads) {
    const int lb = chunk_base + i;
    ids[i] = lb < nblk ? clampi(table[lb], 0, a.num_blocks - 1) : -1;
  }
}

template <int D, int BS>
__device__ __forceinline__ void load_stage(const StagePlan<D, BS>& pl, int64_t stride, const int32_t* ids,
                                           int first, uint4 (&r)[StageLayout<D>::kPerThread]) {
  constexpr int kTiles = kKeys / BS;
  int32_t id[kTiles];
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) id[kt] = ids[first + kt];  // uniform LDS reads
#pragma unroll
  for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
    int b = id[0];
#pragma unroll
    for (int kt = 1; kt < kTiles; ++kt) b = pl.tile[k] == kt ? id[kt] : b;  // select: no dynamic indexing
    r[k] = b >= 0 ? *reinterpret_cast<const uint4*>(pl.base[k] + b * stride) : make_uint4(0, 0, 0, 0);
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
    // keys kk0..kk0+3 go to group 2m, kk0+4..kk0+7 to group 2m+1, each at
    // element (kk0 % 16) / 8 * 4 of its group (m = kk0 / 16).
    const int m = kk0 / 16;
    char* row = vdst + pl.dim[k] * kVRow + ((kk0 % 16) / 8) * 8;
    *reinterpret_cast<uint2*>(row + (2 * m) * 16) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2*>(row + (2 * m + 1) * 16) = make_uint2(x.z, x.w);
  }
}

template <int D, int BS>
__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillSmem<D> sm;
  constexpr int kTileBytes = BS * D * 2;
  // The reference max of a row moves only when the row max exceeds it by
  // more than this (log2 units), so probabilities stay below 2^8 and the
  // accumulators are rescaled only on such moves.
  constexpr float kSlack = 8.f;
  const int s = blockIdx.z;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

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
  const StagePlan<D, BS> plan(a, g);
  const int64_t stride = static_cast<int64_t>(a.num_kv_heads) * kTileBytes;  // bytes per pool block
  constexpr int kTiles = kKeys / BS;
  const int nblk = (L + BS - 1) / BS;

  // This lane's row: token, head, position, validity (lanes l and l+32 share it).
  const int half = lane >> 5;
  int row_pos;
  int64_t row_q;
  bool row_ok;
  {
    const int r = wave * 32 + (lane & 31);
    const int tq = r / G;
    const int j = r - tq * G;
    row_ok = tq < ntok;
    row_pos = row_ok ? pos0 + tq : kend - 1;
    row_q = row_ok ? (static_cast<int64_t>(q0 + tok0 + tq) * a.num_q_heads + g * G + j) * D : -1;
  }

  // Queries: B operand of the QK product, lane holds dims 8*half..+8 of each 16-dim chunk.
  constexpr int kQChunks = D / 16;
  bf16x8 qb[kQChunks];
#pragma unroll
  for (int c = 0; c < kQChunks; ++c) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (row_ok) x = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.q) + row_q + c * 16 + half * 8);
    qb[c] = __builtin_bit_cast(bf16x8, x);
  }

  constexpr int kDimTiles = D / 32;
  float16v acc[kDimTiles];
#pragma unroll
  for (int t = 0; t < kDimTiles; ++t) acc[t] = float16v{};
  float m_run = -INFINITY, l_run = 0.f;

  // Two register sets carry K/V two steps ahead: step j's chunks live in
  // set j % 2 from the load issued during step j - 2 until they are written
  // to LDS at the end of step j - 1.
  uint4 ra[StageLayout<D>::kPerThread], rb[StageLayout<D>::kPerThread];
  int chunk_base = 0;
  fill_ids(a, table, 0, nblk, sm.ids);
  __syncthreads();
  load_stage<D, BS>(plan, stride, sm.ids, 0, ra);
  if (nsteps > 1) load_stage<D, BS>(plan, stride, sm.ids, kTiles, rb);
  store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[0]), plan, 0, L, ra);
  __syncthreads();

  const int key_col = lane & 31;  // key of the QK A operand within the step
  const int k_tile = key_col / BS, k_in = key_col % BS;
  auto step = [&](int st, uint4 (&cur)[StageLayout<D>::kPerThread], uint4 (&nxt)[StageLayout<D>::kPerThread]) {
    // cur: free (step st is in LDS) -> receives step st + 2; nxt: holds step st + 1.
    if (st + 2 < nsteps) {
      if ((st + 2) * kTiles >= chunk_base + kIdChunk) {
        // Every read of the staged ids so far happened before the last barrier.
        chunk_base += kIdChunk;
        fill_ids(a, table, chunk_base, nblk, sm.ids);
        __syncthreads();
      }
      load_stage<D, BS>(plan, stride, sm.ids, (st + 2) * kTiles - chunk_base, cur);
    }
    const char* kl = reinterpret_cast<const char*>(sm.stage[st & 1]);
    const char* vl = kl + StageLayout<D>::kBytes;

    // ---- S^T = K Q^T over the step's 32 keys.
    float16v sc = float16v{};
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
      const bf16x8 ka =
          *reinterpret_cast<const bf16x8*>(kl + k_tile * kTileBytes + ((c * 2 + half) * BS + k_in) * 16);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], sc, 0, 0, 0);
    }

    // ---- online softmax of this lane's 16 scores (keys 8(j/4)+4*half+j%4).
    float x[16];  // scores in log2 units
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = sc[j] * a.scale_log2;
    if (st >= mask_from) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (st * kKeys + 8 * (j / 4) + 4 * half + (j % 4) > row_pos) x[j] = -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, x[j]);
    mx = reduce_pair<true>(mx);
    const bool move = mx > m_run + kSlack;
    const float m_use = move ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_use;
    float sum = 0.f;
    __bf16 pe[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __builtin_amdgcn_exp2f(x[j] - m_use);
      sum += p;
      pe[j] = static_cast<__bf16>(p);
    }
    l_run = l_run * alpha + sum;
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) acc[t] *= alpha;
    }

    // ---- O^T += V^T P^T, two products of 16 keys: product m takes this
    // lane's scores j = 8m..8m+7, i.e. keys 16m+8(i/4)+4*half+i%4, which is
    // how group 2m+half of the V part orders them.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 pb = bf16x8{pe[8 * m], pe[8 * m + 1], pe[8 * m + 2], pe[8 * m + 3],
                               pe[8 * m + 4], pe[8 * m + 5], pe[8 * m + 6], pe[8 * m + 7]};
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vl + (t * 32 + key_col) * kVRow + (2 * m + half) * 16);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[t], 0, 0, 0);
      }
    }

    if (st + 1 < nsteps)
      store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[(st + 1) & 1]), plan, (st + 1) * kKeys, L, nxt);
    __syncthreads();
  };
  for (int st = 0; st < nsteps; st += 2) {
    step(st, ra, rb);
    if (st + 1 < nsteps) step(st + 1, rb, ra);
  }

  // ---- normalise and store: lane holds dims 32t + 8(j/4) + 4*half + j%4 of its row.
  const float l = reduce_pair<false>(l_run);
  if (!row_ok) return;
  const float inv = 1.f / l;
  __bf16* orow = static_cast<__bf16*>(a.out) + row_q;
#pragma unroll
  for (int t = 0; t < kDimTiles; ++t)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      uint32_t w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const __bf16 o0 = static_cast<__bf16>(acc[t][4 * jq + 2 * e] * inv);
        const __bf16 o1 = static_cast<__bf16>(acc[t][4 * jq + 2 * e + 1] * inv);
        w[e] = __builtin_bit_cast(uint16_t, o0) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, o1)) << 16);
      }
      *reinterpret_cast<uint2*>(orow + t * 32 + 8 * jq + 4 * half) = make_uint2(w[0], w[1]);
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
