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
// Plain vector types (not the HIP structs) so staged chunks stay in registers.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

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
  int32_t num_seqs;
  int32_t ntiles;  // query tiles of the longest chunk
  float scale_log2;
};

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2.  Workgroup b runs on XCD b % 8; the mapping below gives every
// workgroup of one (sequence, kv head) pair the same XCD, so the pair's K/V
// tiles, which all its query tiles stream in the same order, are fetched
// into one L2 instead of eight.  Pairs are dealt to the XCDs round-robin
// (pair i to XCD i % 8), and within an XCD a pair's tiles are dispatched
// latest first (they read the most keys).
constexpr int kXcds = 8;

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

// Three stages: step st is consumed (PV) while step st + 1 is consumed
// (QK) and step st + 2 is written.
constexpr int kStages = 3;
template <int D>
struct PrefillSmem {
  u32x4 stage[kStages][StageLayout<D>::kStageBytes / 16];
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
// the same every step, only the block ids change.  A wave's 64 chunks of one
// load are a contiguous 1 KB run inside one (block, kv head) tile (tiles are
// at least 2 KB and aligned to their size), so the tile a chunk belongs to is
// the same across the wave: block ids and tile base addresses are uniform
// (scalar registers) and each lane only adds a 32-bit offset.
template <int D, int BS>
struct StagePlan {
  static constexpr int kTileBytes = BS * D * 2;
  static_assert(kTileBytes >= 64 * 16 * 2, "a wave's chunk run must not straddle tiles");
  const char* kbase;  // K pool + this kv head's tile (add id * stride)
  const char* vbase;  // V pool + this kv head's tile
  int tile[StageLayout<D>::kPerThread];  // tile of the step (0 .. kKeys/BS-1), wave-uniform
  uint32_t src[StageLayout<D>::kPerThread];  // byte offset inside the (block, kv head) tile
  int dst[StageLayout<D>::kPerThread];   // K: byte offset in the K part; V: first key of the chunk in the step
  int dim[StageLayout<D>::kPerThread];   // V: the chunk's dim
  __device__ StagePlan(const PrefillArgs& a, int g) {
    // Chunk k of a thread lies in the K part exactly when k < kPerThread / 2
    // (the K part is the first half of the stage and threads stride it).
    constexpr int kHalf = StageLayout<D>::kPerThread / 2;
    kbase = static_cast<const char*>(a.k_cache) + static_cast<int64_t>(g) * kTileBytes;
    vbase = static_cast<const char*>(a.v_cache) + static_cast<int64_t>(g) * kTileBytes;
#pragma unroll
    for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
      const int ov = (threadIdx.x + kPThreads * (k % kHalf)) * 16;
      tile[k] = __builtin_amdgcn_readfirstlane(ov / kTileBytes);
      const int sv = ov % kTileBytes;
      src[k] = static_cast<uint32_t>(sv);
      dst[k] = k < kHalf ? ov : tile[k] * BS + (sv % (2 * BS)) / 2;  // V: first key of the chunk in the step
      dim[k] = k < kHalf ? 0 : sv / (2 * BS);                        // V tile [D][BS]: 8 keys of one dim
    }
  }
};

// Staged block ids [chunk_base, chunk_base + kIdChunk) of the sequence,
// clamped to the pool.  Past the context the id is 0: such a block is read
// but never used (its keys are masked and its V slots zeroed in LDS).
__device__ __forceinline__ void fill_ids(const PrefillArgs& a, const int32_t* table, int chunk_base, int nblk,
                                         int32_t* ids) {
  for (int i = threadIdx.x; i < kIdChunk; i += kPThreads) {
    const int lb = chunk_base + i;
    ids[i] = lb < nblk ? clampi(table[lb], 0, a.num_blocks - 1) : 0;
  }
}

template <int D, int BS>
__device__ __forceinline__ void load_stage(const StagePlan<D, BS>& pl, int64_t stride, const int32_t* ids,
                                           int first, u32x4 (&r)[StageLayout<D>::kPerThread]) {
  constexpr int kTiles = kKeys / BS;
  constexpr int kHalf = StageLayout<D>::kPerThread / 2;
  int32_t id[kTiles];
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) id[kt] = __builtin_amdgcn_readfirstlane(ids[first + kt]);
#pragma unroll
  for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
    int b = id[0];
#pragma unroll
    for (int kt = 1; kt < kTiles; ++kt) b = pl.tile[k] == kt ? id[kt] : b;  // uniform select
    const char* tb = (k < kHalf ? pl.kbase : pl.vbase) + static_cast<int64_t>(b) * stride;
    r[k] = *reinterpret_cast<const u32x4*>(tb + pl.src[k]);
  }
}

template <int D, int BS>
__device__ __forceinline__ void store_stage(char* dst, const StagePlan<D, BS>& pl, int key_base, int L,
                                            u32x4 (&r)[StageLayout<D>::kPerThread]) {
  constexpr int kHalf = StageLayout<D>::kPerThread / 2;
#pragma unroll
  for (int k = 0; k < kHalf; ++k) *reinterpret_cast<u32x4*>(dst + pl.dst[k]) = r[k];
  char* vdst = dst + StageLayout<D>::kBytes;
  const bool tail = key_base + kKeys > L;  // uniform: only the step holding the context's end
#pragma unroll
  for (int k = kHalf; k < StageLayout<D>::kPerThread; ++k) {
    u32x4 x = r[k];
    const int kk0 = pl.dst[k];  // first key of the chunk within the step (a multiple of 8)
    if (tail) {  // zero V slots at or past the context end
      uint32_t w[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key_base + kk0 + e >= L) w[e / 2] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      x = u32x4{w[0], w[1], w[2], w[3]};
    }
    // keys kk0..kk0+3 go to group 2m, kk0+4..kk0+7 to group 2m+1, each at
    // element (kk0 % 16) / 8 * 4 of its group (m = kk0 / 16).
    const int m = kk0 / 16;
    char* row = vdst + pl.dim[k] * kVRow + ((kk0 % 16) / 8) * 8;
    *reinterpret_cast<u32x2*>(row + (2 * m) * 16) = u32x2{x[0], x[1]};
    *reinterpret_cast<u32x2*>(row + (2 * m + 1) * 16) = u32x2{x[2], x[3]};
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
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, slot = static_cast<int>(blockIdx.x) / kXcds;
  const int pair = xcd + kXcds * (slot / a.ntiles);
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int s = pair / a.num_kv_heads;
  const int g = pair - s * a.num_kv_heads;
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
  const int tile = a.ntiles - 1 - slot % a.ntiles;  // latest tiles first
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

  // Pipeline: during step st the PV product reads LDS stage st % 3, the QK
  // product of step st + 1 reads stage (st + 1) % 3 (its MFMAs overlap this
  // step's exponentials), and step st + 2's K/V, loaded into registers
  // during step st - 1, are written to stage (st + 2) % 3 at the end.  Two
  // register sets alternate: step st loads step st + 3 into one while the
  // other holds step st + 2.
  using Regs = u32x4[StageLayout<D>::kPerThread];
  Regs r0, r1;
  int chunk_base = 0;
  fill_ids(a, table, 0, nblk, sm.ids);
  __syncthreads();
  load_stage<D, BS>(plan, stride, sm.ids, 0, r0);
  store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[0]), plan, 0, L, r0);
  if (nsteps > 1) {
    load_stage<D, BS>(plan, stride, sm.ids, kTiles, r1);
    store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[1]), plan, kKeys, L, r1);
  }
  if (nsteps > 2) load_stage<D, BS>(plan, stride, sm.ids, 2 * kTiles, r0);
  __syncthreads();

  const int key_col = lane & 31;  // key of the QK A operand within the step
  const int k_tile = key_col / BS, k_in = key_col % BS;
  const int k_off = k_tile * kTileBytes + (half * BS + k_in) * 16;
  auto qk = [&](const char* kl) {
    float16v r = float16v{};
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + k_off + c * 2 * BS * 16);
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], r, 0, 0, 0);
    }
    return r;
  };
  auto next = [](int c) { return c == kStages - 1 ? 0 : c + 1; };

  auto step = [&](int st, int cur, Regs& ld, Regs& sv, const float16v& sc, float16v& sn)
                  __attribute__((always_inline)) {
    const int nx1 = next(cur), nx2 = next(nx1);
    if (st + 3 < nsteps) {
      if ((st + 3) * kTiles >= chunk_base + kIdChunk) {
        // Every read of the staged ids so far happened before the last barrier.
        chunk_base += kIdChunk;
        fill_ids(a, table, chunk_base, nblk, sm.ids);
        __syncthreads();
      }
      load_stage<D, BS>(plan, stride, sm.ids, (st + 3) * kTiles - chunk_base, ld);
    }

    // ---- row max of step st (raw scores; the scale is positive, so it
    // commutes with the max and is folded into the exponent below).
    float x[16];  // raw scores of keys 8(j/4)+4*half+j%4
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = sc[j];
    if (st >= mask_from) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (st * kKeys + 8 * (j / 4) + 4 * half + (j % 4) > row_pos) x[j] = -INFINITY;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) mx = fmaxf(mx, x[j]);
    mx = reduce_pair<true>(mx) * a.scale_log2;
    const bool move = mx > m_run + kSlack;
    const float m_use = move ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_use;

    // ---- scores of step st + 1 (on the last step this reads a stage whose
    // contents are unused: in bounds, result dropped).
    sn = qk(reinterpret_cast<const char*>(sm.stage[nx1]));

    __bf16 pe[16];
    float sum;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(x[j], a.scale_log2, -m_use));
      sum = j ? sum + p : p;
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
    const char* vl = reinterpret_cast<const char*>(sm.stage[cur]) + StageLayout<D>::kBytes;
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

    if (st + 2 < nsteps)
      store_stage<D, BS>(reinterpret_cast<char*>(sm.stage[nx2]), plan, (st + 2) * kKeys, L, sv);
    __syncthreads();
  };

  float16v s0 = qk(reinterpret_cast<const char*>(sm.stage[0])), s1;
  int st = 0, cur = 0;
  for (; st + 1 < nsteps; st += 2) {  // unrolled by two: register sets and score sets swap roles
    step(st, cur, r1, r0, s0, s1);
    cur = next(cur);
    step(st + 1, cur, r0, r1, s1, s0);
    cur = next(cur);
  }
  if (st < nsteps) step(st, cur, r1, r0, s0, s1);

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
  // One workgroup per (pair, tile), pairs padded to a multiple of the XCD
  // count; a launch holds at most 2^32 - 1 work-items.
  const int64_t padded = (static_cast<int64_t>(num_seqs) * num_kv_heads + kXcds - 1) / kXcds * kXcds;
  const int64_t max_blocks = UINT32_MAX / kPThreads;
  if (padded > max_blocks || ntiles > max_blocks / padded)
    return pkv::fail(PKV_ERR_INVALID_ARG,
                     "launch too large: %lld (sequence, kv head) pairs x %lld query tiles exceeds %lld workgroups",
                     static_cast<long long>(padded), static_cast<long long>(ntiles), static_cast<long long>(max_blocks));
  const int64_t nblocks = padded * ntiles;
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
  a.num_seqs = num_seqs;
  a.ntiles = static_cast<int32_t>(ntiles);
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<uint32_t>(nblocks));
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
