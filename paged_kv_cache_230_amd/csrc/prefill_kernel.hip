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
//   * One workgroup = 8 waves = one (query tile, kv head, sequence), one
//     workgroup per CU.  The 256 score rows of a tile are (query token,
//     query head) pairs of the G heads sharing the kv head, so every K/V
//     byte staged serves G heads.  Wave w owns rows 32w..32w+31, one per
//     lane pair (l, l+32).  All tiles of one (sequence, kv head) pair run on
//     one XCD, so they share its L2.
//   * Keys advance 32 per step.  The step's K and V block tiles are copied
//     into an 8-stage LDS ring by direct global-to-LDS loads issued 5 steps
//     ahead, as permutations of the pool's 16-byte chunks (layouts at
//     StageLayout); V slots past the context are zeroed in LDS, so unused
//     slots of the last block never reach the products.  A workgroup
//     barrier closes every second step only, so the waves need not run in
//     lockstep.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the step's 32 keys (in slot
//     order) in the rows, the wave's 32 query rows in the columns.  Lane l
//     holds 16 scores of row l%32, keys 16(j/8)+8(l/32)+j%8, so a row's max
//     needs one partner lane, and those scores in that order are the B
//     operand of the PV product: O^T += V^T P^T, again 32x32x16.
//   * The probabilities enter the value product as bf16 high and low parts
//     (two products per tile), so they keep about 2^-17 relative precision;
//     the scores are two chained half dot products summed at the end.
//   * The value product of a step is issued one step after its scores, so
//     each step holds two independent parts: the matrix-core products (the
//     previous step's value product, the next step's scores) and the
//     softmax on the vector ALUs.  The two waves sharing a SIMD run the
//     parts in opposite orders, so that one issues products while the other
//     computes exponentials.
//   * Online softmax per row in the log2 domain; row maxima by the gfx950
//     row swap v_permlane32_swap, not LDS shuffles; the causal mask (a
//     select, never a multiply) only on the steps that reach past the tile's
//     first position.  A row's reference max moves only when its max grows
//     by more than 2^8, so the accumulators are rescaled rarely; the
//     probabilities then stay below 2^8, well inside fp32 and bf16 range.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pkv_status.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float float16v;
// A 16-byte chunk as a plain vector type.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kRows = kPWaves * 32;  // score rows per workgroup (32 per wave)
constexpr int kKeys = 32;                     // keys per step
// Block ids of the tile's key range are staged in LDS this many at a time.
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
  int32_t* status;  // device status word
};

// Sets a PKV_DEV_* flag in the device status word.
__device__ __forceinline__ void report(int32_t* status, int32_t flag) {
  __hip_atomic_fetch_or(status, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2.  Workgroup b runs on XCD b % 8; the mapping below gives every
// workgroup of one (sequence, kv head) pair the same XCD, so the pair's K/V
// tiles, which all its query tiles stream in the same order, are fetched
// into one L2 instead of eight.  Pairs are dealt to the XCDs round-robin
// (pair i to XCD i % 8), and within an XCD a pair's tiles are dispatched
// latest first (they read the most keys).
constexpr int kXcds = 8;

// One step's K and V in LDS, each a copy of the step's kKeys/BS pool tiles
// whose 16-byte chunks (8 bf16) are permuted, never split, so the copy is
// done by direct global-to-LDS loads (global_load_lds_dwordx4: each lane
// names its source chunk, the wave's 64 chunks land contiguously).
//   K part: [kKeys/BS tiles][D/8][BS slots][8]; slot s holds key pi(s),
//     pi swapping bits 2 and 3 of s.  Lane l of a QK A operand reads slot
//     l % 32, so the product's output rows come out in key order pi, which
//     makes a lane's 16 scores the keys 16(j/8) + 8(l/32) + j%8: per 16-key
//     half, 8 consecutive keys, exactly the B operand of the PV product.
//     Each 16-lane quarter of an A read is a contiguous 256-byte run.
//   V part: [kKeys/BS tiles][D][BS/8 chunks][8], the pool's [D][BS] tile
//     with the chunks of row d XOR-swizzled by vswz(d) so the 16 dims a
//     quarter-wave reads hit distinct banks.
template <int D>
struct StageLayout {
  static constexpr int kBytes = kKeys * D * 2;  // bytes of the K or the V part
  static constexpr int kStageBytes = 2 * kBytes;
  static constexpr int kPerThread = kStageBytes / 16 / kPThreads;  // DMA loads per thread per stage
  static_assert((kStageBytes / 16) % kPThreads == 0, "stage must split evenly over the threads");
};

// Stage ring: during step st the PV product reads stage st - 1, the QK product
// of step st + 1 reads stage st + 1, and the loads of step st + kAhead are
// issued into the stage step st - kBarrierEvery - 1 used (all modulo
// kStages); the stages in between are landing.
constexpr int kStages = 8;
// A workgroup barrier closes every kBarrierEvery-th step; between barriers
// the waves may run up to kBarrierEvery - 1 steps apart, and a stage's last
// reader is the value product one step after its scores, so a stage may be
// reloaded only kBarrierEvery + 1 steps after its scores were computed.
constexpr int kBarrierEvery = 2;
constexpr int kAhead = kStages - kBarrierEvery - 1;
static_assert(kAhead >= kBarrierEvery + 1, "the stage read next must have landed at each barrier");
template <int D>
struct PrefillSmem {
  u32x4 stage[kStages][StageLayout<D>::kStageBytes / 16];
  int32_t ids[kIdChunk];
};

typedef __attribute__((address_space(3))) void* LdsPtr;

__device__ __forceinline__ int pi_slot(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

template <int BS>
__device__ __forceinline__ int vswz(int d) {
  constexpr int n = BS / 8;  // chunks per V row
  return (d * n / 8) % n;
}

// s_waitcnt with vmcnt(n), lgkmcnt(0) and no wait on export counts (the
// 6-bit vmcnt field is split: bits 3:0 and 15:14).
template <int kN>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(kN >= 0 && kN < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier after this wave's LDS accesses and all but its newest kN
// global-to-LDS loads have completed.  No memory fence (a fence would also
// wait for the loads still in flight for later stages); the empty asm
// statements keep the compiler from moving memory accesses across it.
template <int kN>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  wait_vm_lgkm0<kN>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// Barrier once all but the loads of this wave's newest n steps have landed
// (n uniform, 0 <= n <= kN; the wait count must be an immediate).
template <int kPer, int kN>
__device__ __forceinline__ void barrier_after_steps(int n) {
  if constexpr (kN == 0) {
    stage_barrier<0>();
  } else {
    if (n >= kN)
      stage_barrier<kN * kPer>();
    else
      barrier_after_steps<kPer, kN - 1>(n);
  }
}

// Where each of a thread's DMA loads comes from and goes to; the same every
// step, only the block ids change.  Load k of thread t fills LDS chunk
// k * kPThreads + t of the stage, so a wave's load is a contiguous 1 KB run
// inside one (block, kv head) tile (tiles are at least 2 KB and aligned to
// their size): block ids, tile bases and LDS addresses are wave-uniform and
// each lane adds a 32-bit source offset.
template <int D, int BS>
struct StagePlan {
  static constexpr int kTileBytes = BS * D * 2;
  static constexpr int kTileChunks = kTileBytes / 16;
  static constexpr int kPartChunks = StageLayout<D>::kBytes / 16;  // chunks of the K (or V) part
  static_assert(kTileChunks % 64 == 0 && kPartChunks % 64 == 0, "a wave's chunk run must not straddle tiles");
  const char* kbase;  // K pool + this kv head's tile (add id * stride)
  const char* vbase;  // V pool + this kv head's tile
  int tile[StageLayout<D>::kPerThread];      // tile of the step (0 .. kKeys/BS-1), wave-uniform
  bool vpart[StageLayout<D>::kPerThread];    // the load fills the V part, wave-uniform
  uint32_t src[StageLayout<D>::kPerThread];  // byte offset inside the (block, kv head) tile
  int lds[StageLayout<D>::kPerThread];       // byte offset of the wave's run in the stage, wave-uniform
  __device__ StagePlan(const PrefillArgs& a, int g) {
    kbase = static_cast<const char*>(a.k_cache) + static_cast<int64_t>(g) * kTileBytes;
    vbase = static_cast<const char*>(a.v_cache) + static_cast<int64_t>(g) * kTileBytes;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
      const int p = k * kPThreads + static_cast<int>(threadIdx.x);  // chunk of the stage
      const bool is_v = p >= kPartChunks;
      const int pp = is_v ? p - kPartChunks : p;
      vpart[k] = __builtin_amdgcn_readfirstlane(static_cast<int>(is_v)) != 0;
      tile[k] = __builtin_amdgcn_readfirstlane(pp / kTileChunks);
      const int r = pp % kTileChunks;
      int chunk;
      if (!is_v) {  // K: r = (d/8) * BS + slot
        chunk = (r / BS) * BS + pi_slot(r % BS);
      } else {      // V: r = d * (BS/8) + swizzled chunk
        constexpr int n = BS / 8;
        const int d = r / n;
        chunk = d * n + ((r % n) ^ vswz<BS>(d));
      }
      src[k] = static_cast<uint32_t>(chunk) * 16u;
      lds[k] = (k * kPThreads + wave * 64) * 16;
    }
  }
};

// Staged block ids [chunk_base, chunk_base + kIdChunk) of the sequence,
// clamped to the pool (an id outside it is reported).  Past the context the
// id is 0: such a block is read but never used (its keys are masked and its
// V slots zeroed in LDS).
__device__ __forceinline__ void fill_ids(const PrefillArgs& a, const int32_t* table, int chunk_base, int nblk,
                                         int32_t* ids) {
  for (int i = threadIdx.x; i < kIdChunk; i += kPThreads) {
    const int lb = chunk_base + i;
    int id = 0;
    if (lb < nblk) {
      const int raw = table[lb];
      id = clampi(raw, 0, a.num_blocks - 1);
      if (id != raw) report(a.status, PKV_DEV_BAD_BLOCK_ID);
    }
    ids[i] = id;
  }
}

// One step's block ids as read from LDS (the same in every lane).  They are
// read a step before their loads are issued and made scalar only then, so
// the LDS read completes behind other work instead of stalling the wave.
template <int BS>
struct StepIds {
  int32_t v[kKeys / BS];
  __device__ __forceinline__ void read(const int32_t* ids, int first) {
#pragma unroll
    for (int kt = 0; kt < kKeys / BS; ++kt) v[kt] = ids[first + kt];
  }
};

// Issue the DMA loads of one step into a stage.
template <int D, int BS>
__device__ __forceinline__ void load_stage(u32x4* stage, const StagePlan<D, BS>& pl, int64_t stride,
                                           const StepIds<BS>& ids) {
  constexpr int kTiles = kKeys / BS;
  int32_t id[kTiles];
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) id[kt] = __builtin_amdgcn_readfirstlane(ids.v[kt]);
#pragma unroll
  for (int k = 0; k < StageLayout<D>::kPerThread; ++k) {
    int b = id[0];
#pragma unroll
    for (int kt = 1; kt < kTiles; ++kt) b = pl.tile[k] == kt ? id[kt] : b;  // uniform select
    const char* tb = (pl.vpart[k] ? pl.vbase : pl.kbase) + static_cast<int64_t>(b) * stride;
    __builtin_amdgcn_global_load_lds(tb + pl.src[k], (LdsPtr)(reinterpret_cast<char*>(stage) + pl.lds[k]), 16, 0, 0);
  }
}

// Zero the V entries of keys at or past the context end L in a landed stage
// (the stage holding the context's end; its unused slots may hold anything,
// and a zero probability times a NaN would still be NaN).
template <int D, int BS>
__device__ void zero_v_tail(u32x4* stage, int key_base, int L) {
  constexpr int kTileBytes = BS * D * 2;
  constexpr int n = BS / 8;
  char* v = reinterpret_cast<char*>(stage) + StageLayout<D>::kBytes;
  for (int i = threadIdx.x; i < D * kKeys; i += kPThreads) {
    const int d = i / kKeys, key = i % kKeys;
    if (key_base + key >= L) {
      const int chunk = d * n + (((key % BS) / 8) ^ vswz<BS>(d));
      *reinterpret_cast<uint16_t*>(v + (key / BS) * kTileBytes + chunk * 16 + (key % 8) * 2) = 0;
    }
  }
}

template <int D, int BS>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a) {
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

  const int Lraw = a.context_lens[s];
  const int L = clampi(Lraw, 0, a.max_blocks_per_seq * BS);
  int q0 = a.query_start[s];
  const int Craw = a.query_start[s + 1] - q0;
  int C = Craw;
  if (q0 < 0 || q0 > a.num_tokens) C = 0;
  C = clampi(C, 0, L < a.max_query_len ? L : a.max_query_len);
  if (q0 + C > a.num_tokens) C = a.num_tokens - q0;
  if (slot % a.ntiles == 0 && threadIdx.x == 0) {  // one workgroup per (sequence, kv head) reports
    if (Lraw != L) report(a.status, PKV_DEV_BAD_LENGTH);
    if (C != Craw) report(a.status, PKV_DEV_BAD_QUERY_START);
  }
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

  // Pipeline (see kStages, kBarrierEvery): the loads of step st + kAhead are
  // issued at the top of step st; a barrier waits for this wave's loads of
  // the stages the QK products read before the next barrier (later steps'
  // may still be in flight) and so publishes them.
  constexpr int kPer = StageLayout<D>::kPerThread;
  int chunk_base = 0;
  fill_ids(a, table, 0, nblk, sm.ids);
  __syncthreads();
  StepIds<BS> ids;  // ids of the step whose loads are issued next
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    if (k < nsteps) {
      ids.read(sm.ids, k * kTiles);
      load_stage<D, BS>(sm.stage[k], plan, stride, ids);
    }
  }
  if (kAhead < nsteps) ids.read(sm.ids, kAhead * kTiles);  // for the loads issued in step 0
  const bool tail = nsteps * kKeys > L;  // the last step reaches past the context end
  // stages 0 .. kBarrierEvery landed; later steps up to min(kAhead, nsteps) - 1 may be in flight
  constexpr int kInFlight = kAhead - kBarrierEvery - 1;  // steps a barrier lets stay in flight
  barrier_after_steps<kPer, kInFlight>((nsteps < kAhead ? nsteps : kAhead) - kBarrierEvery - 1);

  const int key_col = lane & 31;  // QK A operand slot of this lane
  const int k_tile = key_col / BS, k_in = key_col % BS;
  const int k_off = k_tile * kTileBytes + (half * BS + k_in) * 16;
  // The dot product runs as two chained halves (dims 0..D/2-1 and
  // D/2..D-1) summed at the end: with logits in the hundreds, rounding every
  // partial sum of one long chain to fp32 moves the softmax weights of
  // near-tied keys enough to show in outputs near zero.
  auto qk = [&](const char* kl) {
    float16v r0 = float16v{}, r1 = float16v{};
#pragma unroll
    for (int c = 0; c < kQChunks; ++c) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + k_off + c * 2 * BS * 16);
      if (c < kQChunks / 2)
        r0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], r0, 0, 0, 0);
      else
        r1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[c], r1, 0, 0, 0);
    }
    return r0 + r1;
  };
  // V operand offsets: PV product m, dim tile t; lane dim 32t + l%32 reads
  // keys 16m + 8(l/32) .. +7, i.e. chunk (16m + 8 half) / 8 of its row.
  int v_off[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int key = 16 * m + 8 * half;
    v_off[m] = StageLayout<D>::kBytes + (key / BS) * kTileBytes +
               (key_col * (BS / 8) + (((key % BS) / 8) ^ vswz<BS>(key_col))) * 16;
  }
  static_assert(32 % (8 / (BS / 8)) == 0, "the V swizzle repeats within 32 dims");

  // Probabilities of the step whose value product is issued next, as bf16
  // pairs: high parts and the bf16 roundings of the remainders (keys
  // 16(j/8) + 8*half + j%8 for j = 2*i, 2*i + 1).
  uint32_t pe2[8], pr2[8];
  // The rescale of the accumulators that the previous step's row max asks
  // for; it is applied just before that step's value product.
  float alpha_prev = 1.f;
  bool move_prev = false;

  // O^T += V^T P^T for the step whose scores gave pe2/pr2, from the V part
  // of its stage: two products of 16 keys; product m takes this lane's
  // scores j = 8m..8m+7, keys 16m + 8*half + i, the B operand's k order; the
  // V operand of lane l holds the same keys of dim 32t + l%32.  The high and
  // low parts of P each take one product with the same V operand.
  auto pv = [&](const char* sl, const uint32_t (&pe)[8], const uint32_t (&pr)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pe[4 * m], pe[4 * m + 1], pe[4 * m + 2], pe[4 * m + 3]});
      const bf16x8 pbl = __builtin_bit_cast(bf16x8, u32x4{pr[4 * m], pr[4 * m + 1], pr[4 * m + 2], pr[4 * m + 3]});
      // All high-part products, then all low-part ones: a product that adds
      // to an accumulator then trails the previous one on it by kDimTiles
      // issues, not one (+1.5 %).
      bf16x8 va[kDimTiles];
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) va[t] = *reinterpret_cast<const bf16x8*>(sl + v_off[m] + t * 32 * (BS / 8) * 16);
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pb, acc[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], pbl, acc[t], 0, 0, 0);
    }
  };
  auto rescale_prev = [&]() __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(move_prev)) {  // rare
#pragma unroll
      for (int t = 0; t < kDimTiles; ++t) acc[t] *= alpha_prev;
    }
  };

  // Step st: scores of step st (sc) -> probabilities; scores of step st + 1
  // (sn); the value product of step st - 1.  The value product trails its
  // scores by a step so that one basic block holds both products and the
  // softmax of the step, which share no operands: the wave's matrix-core
  // and vector-ALU work can then overlap.
  auto step = [&](auto with_pv, auto mfma_first, int st, int cur, const float16v& sc, float16v& sn)
                  __attribute__((always_inline)) {
    const int nx1 = (cur + 1) % kStages, nxa = (cur + kAhead) % kStages, prv = (cur + kStages - 1) % kStages;
    if (st + kAhead < nsteps) {
      load_stage<D, BS>(sm.stage[nxa], plan, stride, ids);
      if (st + kAhead + 1 < nsteps) {
        if ((st + kAhead + 1) * kTiles >= chunk_base + kIdChunk) {
          __syncthreads();  // every wave has read the ids of its steps so far
          chunk_base += kIdChunk;
          fill_ids(a, table, chunk_base, nblk, sm.ids);
          __syncthreads();
        }
        ids.read(sm.ids, (st + kAhead + 1) * kTiles - chunk_base);  // its loads are issued a step later
      }
    }

    // Raw scores of keys 16(j/8) + 8*half + j%8, masked past the row's
    // position (a select, never a multiply).  The branches come before the
    // products so that they do not split the products off the softmax.
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = sc[j];
    if (st >= mask_from) {
      const int lim = row_pos - st * kKeys - 8 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (16 * (j / 8) + (j % 8) > lim) x[j] = -INFINITY;
    }
    if constexpr (decltype(with_pv)::value) rescale_prev();

    uint32_t pe_prev[8], pr_prev[8];  // the probabilities of step st - 1
#pragma unroll
    for (int j2 = 0; j2 < 8; ++j2) {
      pe_prev[j2] = pe2[j2];
      pr_prev[j2] = pr2[j2];
    }
    // The matrix-core products of the step: the value product of step
    // st - 1 and the scores of step st + 1 (on the last step this reads a
    // stage whose contents are unused: in bounds, result dropped).
    auto products = [&]() __attribute__((always_inline)) {
      if constexpr (decltype(with_pv)::value) pv(reinterpret_cast<const char*>(sm.stage[prv]), pe_prev, pr_prev);
      sn = qk(reinterpret_cast<const char*>(sm.stage[nx1]));
    };
    // The vector-ALU part: the softmax of step st.
    auto softmax = [&]() __attribute__((always_inline)) {
      // ---- row max (raw scores; the scale is positive, so it commutes
      // with the max and is folded into the exponent below).
      float mx = fmaxf(x[0], x[1]);
#pragma unroll
      for (int j = 2; j < 16; ++j) mx = fmaxf(mx, x[j]);
      mx = reduce_pair<true>(mx) * a.scale_log2;
      const bool move = mx > m_run + kSlack;
      const float m_use = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_use;
      // Each probability enters the value product as a bf16 high part and
      // the bf16 rounding of the remainder, so it is carried to about 2^-17
      // relative precision (one bf16 alone, 2^-9, leaves outputs near zero
      // with relative errors of tens of percent).
      // Converted in pairs: one packed conversion gives two high parts,
      // whose fp32 values are the packed word shifted or masked; one more
      // gives the two low parts.
      float sum;
#pragma unroll
      for (int j2 = 0; j2 < 8; ++j2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(x[2 * j2], a.scale_log2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(x[2 * j2 + 1], a.scale_log2, -m_use));
        sum = j2 ? sum + p0 + p1 : p0 + p1;
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
        const float h0 = __builtin_bit_cast(float, hi << 16), h1 = __builtin_bit_cast(float, hi & 0xFFFF0000u);
        pe2[j2] = hi;
        pr2[j2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0 - h0, p1 - h1}, bf16x2));
      }
      // Keep the probabilities in this step: the compiler would otherwise
      // sink their computation into the next step, next to their only use.
#pragma unroll
      for (int j2 = 0; j2 < 8; ++j2) asm volatile("" : "+v"(pe2[j2]), "+v"(pr2[j2]));
      l_run = l_run * alpha + sum;
      alpha_prev = alpha;
      move_prev = move;
    };
    // The two waves sharing a SIMD (waves w and w + 4) take the two parts in
    // opposite orders, so that after each barrier one issues matrix-core
    // products while the other runs its softmax on the vector ALUs.  The
    // scheduling barrier keeps the instruction scheduler from interleaving
    // the parts within a wave (+1 % against one order for all waves).
    if constexpr (decltype(mfma_first)::value) {
      products();
      __builtin_amdgcn_sched_barrier(0);
      softmax();
    } else {
      softmax();
      __builtin_amdgcn_sched_barrier(0);
      products();
    }

    // The barrier closing step st (every kBarrierEvery-th step) leaves
    // stages up to st + kBarrierEvery + 1 landed, which the QK products of
    // the steps until the next barrier read; steps after that up to
    // min(st + kAhead, nsteps - 1) may be in flight.
    if ((st + 1) % kBarrierEvery == 0)
      barrier_after_steps<kPer, kInFlight>((nsteps - 1 - st < kAhead ? nsteps - 1 - st : kAhead) - kBarrierEvery - 1);
  };

  using no_pv = std::integral_constant<bool, false>;
  using with_pv = std::integral_constant<bool, true>;
  auto run_steps = [&](auto mfma_first) __attribute__((always_inline)) {
    float16v s0 = qk(reinterpret_cast<const char*>(sm.stage[0])), s1;
    step(no_pv{}, mfma_first, 0, 0, s0, s1);
    int st = 1, cur = 1;
    for (; st + 1 < nsteps; st += 2) {  // unrolled by two: the score sets swap roles
      step(with_pv{}, mfma_first, st, cur, s1, s0);
      cur = (cur + 1) % kStages;
      step(with_pv{}, mfma_first, st + 1, cur, s0, s1);
      cur = (cur + 1) % kStages;
    }
    if (st < nsteps) {
      step(with_pv{}, mfma_first, st, cur, s1, s0);
      cur = (cur + 1) % kStages;
    }
    return cur;
  };
  const int cur = (wave & 4) ? run_steps(std::integral_constant<bool, false>{})
                             : run_steps(std::integral_constant<bool, true>{});
  // ---- the last step's value product; if the context ends inside that
  // step, its V slots past the end are zeroed first (no wave reads that
  // stage's V part before this point, and no load is in flight into it).
  const int last = (cur + kStages - 1) % kStages;
  if (tail) {
    zero_v_tail<D, BS>(sm.stage[last], (nsteps - 1) * kKeys, L);
    stage_barrier<63>();
  }
  rescale_prev();
  pv(reinterpret_cast<const char*>(sm.stage[last]), pe2, pr2);

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
  if (int32_t e = pkv::device_status_ptr(&a.status)) return e;
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
