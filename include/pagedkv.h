/*
 * pagedkv.h -- C ABI of the paged KV-cache decode library (gfx950 / MI355X).
 *
 * The library implements the data-parallel hot path of PagedAttention:
 *   - a host block manager (free pool, reference counts, copy-on-write),
 *   - the copy-on-write block copy and the cache append on the GPU,
 *   - single-query decode attention that reads K/V through per-sequence
 *     block tables, split over context partitions and merged by log-sum-exp.
 *
 * Sources (page title, section):
 *   [gloss]  "PagedAttention" (ayinedjimi-consultants.fr glossary), Définition
 *   [sheet]  "PagedAttention — Gestion mémoire pour LLM à long contexte"
 *            (analyticslegends.ai), Pourquoi c'est important / Points clés /
 *            Termes employés sur cette page
 *   [pl]     "PagedAttention" (robocikowo.com), Jak działa / Komponenty /
 *            Złożoność obliczeniowa
 *   [aitalk] "PagedAttention et RadixAttention : parlons de KV Cache"
 *            (aitalk.it), section "PagedAttention : la mémoire comme un
 *            système d'exploitation", steps 1-4 and closing paragraph
 *
 * General conventions
 *   - Every function returns an int32 status (PKV_OK = 0, negative on
 *     error) unless stated; pkv_last_error() then describes the failure for
 *     the calling thread.
 *   - Device pointers are plain device addresses (e.g. from hipMalloc or a
 *     framework tensor).  The caller owns every buffer, including the
 *     decode workspace; the library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Device entry points only enqueue work on it and return; ordering is
 *     the stream's.  They validate sizes and pointers on the host before
 *     launching; device-side indices (slots, block ids, lengths) are range
 *     checked in the kernels so bad values never touch memory outside the
 *     buffers (the affected results are then unspecified).
 *   - Device entry points are re-entrant.  A block manager handle must be
 *     used by one thread at a time.
 *
 * Pool format (both pools hold one layer; the caller allocates them):
 *   x = 16 / sizeof(element)  (4 for fp32, 8 for bf16)
 *   K pool: [num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *           token o of block b, kv head h, dimension i is element
 *           [b][h][i / x][o][i % x]
 *   V pool: [num_blocks][num_kv_heads][head_dim][block_size]
 *           element [b][h][i][o]
 *   Slot s addresses token offset s % block_size of block s / block_size.
 *   The pages fix fixed-size blocks of token slots, 16 or 32 per block, per
 *   layer, placed anywhere in GPU memory ([gloss] Définition; [sheet] Points
 *   clés; [pl] Jak działa; [aitalk] step 1); the byte layout inside a block is
 *   this library's choice: every (block, kv head) tile is contiguous and the
 *   layout gives whole-wavefront contiguous 16-byte loads in the decode
 *   kernel's matrix-core operand order.
 *
 * Supported shapes: dtype PKV_F32 or PKV_BF16; head_dim 64 or 128;
 * block_size 16 or 32; num_q_heads a multiple of num_kv_heads with group
 * size G = num_q_heads / num_kv_heads <= 8 (bf16) or <= 16 (fp32).
 * Query head h uses kv head h / G.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1)   /* bad size, pointer, alignment or id     */
#define PKV_ERR_OUT_OF_BLOCKS (-2) /* free pool cannot satisfy the request   */
#define PKV_ERR_UNKNOWN_SEQ (-3)   /* sequence id not registered             */
#define PKV_ERR_DEVICE (-4)        /* a HIP call or kernel launch failed     */
#define PKV_ERR_UNSUPPORTED (-5)   /* dtype/head_dim/block_size/G not built  */
#define PKV_ERR_CAPACITY (-6)      /* caller's output buffer too small       */

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Flags of the device status word (pkv_device_status).  A kernel that
 * meets a device-side index outside its range skips (or, for decode
 * reads, clamps into the buffers) the access it names and ORs one of these
 * into the word of the GPU it runs on; results that depend on the value
 * are then unspecified, but no access leaves the buffers. */
#define PKV_DEV_BAD_BLOCK_ID 1    /* a block-table entry in use outside [0, num_blocks) */
#define PKV_DEV_BAD_LENGTH 2      /* a context length outside [0, max_context_len]     */
#define PKV_DEV_BAD_SLOT 4        /* an append slot at or past num_blocks * block_size  */
#define PKV_DEV_BAD_PAIR 8        /* a copy or swap pair naming a block outside a pool  */
#define PKV_DEV_BAD_RECORD 16     /* a staged table update outside the device table     */
#define PKV_DEV_BAD_QUERY_START 32 /* prefill query_start not rising in [0, num_tokens] */

/* Flags of the decode calls (paged_attention_decode*).                    */
/* PKV_DECODE_SHARED_BLOCKS: several sequences of the batch read the same  */
/*   blocks (shared prompt prefixes, forked samples: "PagedAttention et    */
/*   RadixAttention : parlons de KV Cache", step 4, and the part on        */
/*   automatic prefix caching).  The kernel then reads K/V through the     */
/*   caches and keeps each kv head's workgroups on one XCD, so a shared    */
/*   block fetched for one sequence serves the others from that XCD's L2.  */
/*   Without the flag, K/V are streamed with non-temporal loads, which do  */
/*   not fill the caches: faster when every block is read once per call.   */
/*   Results are identical either way; the flag only chooses the faster     */
/*   schedule.  pkv_bm_num_shared tells whether a block manager's pool     */
/*   holds shared blocks.                                                  */
#define PKV_DECODE_SHARED_BLOCKS 1u

/* Message for the last failing call on this thread ("" if none).  The
 * string is owned by the library and valid until the thread's next call. */
const char* pkv_last_error(void);

/* Measurement helper: reads `bytes` (a multiple of 16) of device memory at
 * `buf` (16-byte aligned) once with a plain streaming kernel of
 * min(bytes / 4096, sink_words) workgroups, each folding what it read into
 * one word of `sink` (device uint32 [sink_words]).  Timing it gives the
 * HBM read rate this GPU reaches for a simple stream, the practical ceiling
 * beside the nominal peak for the bandwidth-bound decode kernel ([pl]
 * Złożoność obliczeniowa: the kernel is bound by HBM bandwidth).
 * Asynchronous on `stream`. */
int32_t pkv_stream_read(const void* buf, size_t bytes, void* sink, int32_t sink_words, void* stream);

/* Measurement helper: reads num_tiles tiles of tile_bytes (a positive
 * multiple of 1024) at base + ids[i] * tile_bytes once each, with the same
 * non-temporal 16-byte loads as pkv_stream_read; ids (device int32
 * [num_tiles]) are clamped to [0, max_tiles), so every read stays inside
 * base's max_tiles tiles (base 16-byte aligned).  Each wave reads whole
 * tiles of a contiguous share of the list; at most sink_words workgroups,
 * each folding what it read into one word of `sink` (device uint32
 * [sink_words]).  Run over the (block, kv head) tiles a decode call reads,
 * it gives the rate at which those very tiles can be streamed without any
 * arithmetic: the ceiling of the bandwidth-bound decode kernel for that
 * access pattern ([pl] Złożoność obliczeniowa; [aitalk] step 2: the blocks
 * are scattered through the pool).  Errors: null pointers, misalignment,
 * bad sizes (PKV_ERR_INVALID_ARG), launch failure (PKV_ERR_DEVICE).
 * Asynchronous on `stream`. */
int32_t pkv_tile_read(const void* base, size_t tile_bytes, size_t max_tiles, const int32_t* ids, int64_t num_tiles,
                      void* sink, int32_t sink_words, void* stream);

/* Measurement helper: launches `workgroups` workgroups of 512 threads (8
 * waves); every wave issues `iters` x 16 bf16 matrix products
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands into four
 * independent accumulators, and every thread writes one float to
 * sink[workgroup * 512 + thread] (device float [workgroups * 512], 4-byte
 * aligned, owned by the caller).  Flops issued: workgroups * 8 * iters * 16 *
 * 32768.  Timing it gives the bf16 matrix-core rate this GPU sustains (it
 * lowers its clock under such load), the practical ceiling beside the
 * nominal peak for the matrix-core-bound chunked prefill ([aitalk] the
 * part on the two independent problems: prefill computes the prompt's K/V
 * and attention).  Errors: null or misaligned sink, workgroups <= 0 or
 * above 8388607 (2^32 - 1 work-items), iters < 0 (PKV_ERR_INVALID_ARG),
 * launch failure (PKV_ERR_DEVICE).
 * Asynchronous on `stream`. */
int32_t pkv_mfma_rate(void* sink, int32_t workgroups, int32_t iters, void* stream);

/* Library interface version (major * 100 + minor). */
int32_t pkv_version(void);

/* Device status word of the current GPU: waits for `stream`, stores the
 * OR of the PKV_DEV_* flags that kernels have set since the word was last
 * cleared in *flags_out (0 = every device-side index was in range), and
 * clears the word when `clear` is nonzero.  The word is shared by every
 * call on that GPU; work running on other streams meanwhile may set a flag
 * between the read and the clear.  Not for use under graph capture (it
 * synchronises).  Errors: PKV_ERR_INVALID_ARG (null flags_out),
 * PKV_ERR_DEVICE (no device, a failed copy). */
int32_t pkv_device_status(void* stream, int32_t clear, int32_t* flags_out);

/* ------------------------------------------------------------------ */
/* Cache append ([aitalk] step 3: the cache grows one slot at a time; a  */
/* token is written into the slot the block manager reserved for it).    */
/*                                                                        */
/* k_new, v_new : device, [num_tokens][num_kv_heads][head_dim], dtype dt, */
/*                16-byte aligned rows                                    */
/* k_cache, v_cache : device pools in the format above, num_blocks blocks */
/* slot_mapping : device int32 [num_tokens]; slot < 0 skips the token;    */
/*                slots must be distinct (duplicates race); a slot at or  */
/*                past num_blocks * block_size is skipped and sets        */
/*                PKV_DEV_BAD_SLOT                                        */
/* Writes K/V of each token into its slot; every other byte is untouched. */
/* num_tokens == 0 is a no-op.                                            */
int32_t paged_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks, pkv_dtype dt,
                        void* stream);

/* ------------------------------------------------------------------ */
/* Copy-on-write block copy ([pl] Komponenty: reference counting with    */
/* lazy duplication; [aitalk] step 4: a shared block is copied only when */
/* a sequence diverges from the others).                                 */
/*                                                                        */
/* src_dst : device int32 [num_pairs][2] = (source block, destination     */
/*           block); whole blocks (all kv heads, all slots) of both pools */
/*           are copied.  Pairs run concurrently: no destination may be a */
/*           source or destination of another pair (the block manager's   */
/*           pairs satisfy this).  num_pairs == 0 is a no-op.             */
int32_t paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t num_pairs,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             pkv_dtype dt, void* stream);

/* Whole-block copies between two pools of the same format (the device    */
/* pool and a host swap pool, either way): for each pair (s, d),          */
/* dst[d] = src[s] for K and V, all kv heads ([sheet] Page eviction).     */
/* Each of src_k, src_v, dst_k, dst_v may be device memory or pinned host */
/* memory (read or written in place over the bus; pageable host memory is */
/* rejected).  pairs: device (or pinned host) int32 [num_pairs][2]; pairs */
/* naming blocks outside [0, src_num_blocks) or [0, dst_num_blocks) are  */
/* skipped.  Asynchronous on `stream`.                                     */
int32_t paged_kv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* pairs,
                             int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t src_num_blocks, int32_t dst_num_blocks, pkv_dtype dt, void* stream);

/* ------------------------------------------------------------------ */
/* Decode attention ([pl] Jak działa and Komponenty: an attention kernel  */
/* that reads a non-contiguous cache through the block table; [aitalk]   */
/* step 2 and closing paragraph: the sequence appears contiguous and the */
/* attention result is unchanged by paging).                             */
/*                                                                        */
/* For each sequence s (context length L = context_lens[s], the number   */
/* of cached tokens to attend to, including one appended this step) and  */
/* query head h (kv head g = h / G):                                      */
/*   out[s][h] = sum_t softmax_t(scale * <q[s][h], K_t[g]>) V_t[g],       */
/* t over the first L slots named by block_tables[s].  L == 0 gives a    */
/* zero row.  Scores, softmax and the weighted sum are computed in fp32;  */
/* bf16 outputs are rounded to nearest-even.                             */
/*                                                                        */
/* out, q        : device, [num_seqs][num_q_heads][head_dim], dtype dt    */
/* k_cache, v_cache : device pools, num_blocks blocks                     */
/* block_tables  : device int32 [num_seqs][max_blocks_per_seq]; entries   */
/*                 past ceil(L / block_size) are not read                 */
/* context_lens  : device int32 [num_seqs], each in [0, max_context_len]; */
/*                 a value outside is clamped into that range and sets    */
/*                 PKV_DEV_BAD_LENGTH; a table entry in use outside       */
/*                 [0, num_blocks) reads block 0 and sets                 */
/*                 PKV_DEV_BAD_BLOCK_ID                                   */
/* max_context_len : host upper bound on context_lens, <=                 */
/*                 max_blocks_per_seq * block_size                        */
/* scale         : logit scale (usually 1/sqrt(head_dim))                 */
/* partition_size: 0 (default) splits the work over one round of the     */
/*                 workgroups the GPU holds at once; > 0 asks for about   */
/*                 that many tokens per workgroup (num_seqs *             */
/*                 max_context_len / partition_size workgroups per kv     */
/*                 head; a value >= that product means one workgroup per  */
/*                 kv head and no sequence is split).  Results differ     */
/*                 only by fp32 rounding between splits.                  */
/* workspace     : device scratch, at least                               */
/*                 paged_attention_workspace_bytes(...) bytes, 256-byte   */
/*                 aligned, required whenever num_seqs > 0: it holds, per */
/*                 (sequence, kv head), the record of the pieces a split  */
/*                 sequence was cut into, and the pieces' partials.  Any  */
/*                 content is accepted (each call writes what it reads);  */
/*                 calls sharing a workspace must be ordered on one       */
/*                 stream.                                                */
/* flags         : 0 or PKV_DECODE_SHARED_BLOCKS (cache policy, above);   */
/*                 other bits fail with PKV_ERR_INVALID_ARG               */
/*                                                                        */
/* Work distribution (balanced split): for each kv head the blocks of all */
/* sequences form one list in which every sequence is also charged       */
/* paged_attention_segment_cost(block_size) blocks of fixed work; each of */
/* the N workgroups of that head takes an equal contiguous range of it.   */
/* A range covering a whole sequence writes its rows; pieces of a split   */
/* sequence write partials that a second kernel merges by log-sum-exp.    */
int32_t paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                               float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                               pkv_dtype dt, uint32_t flags, void* stream);

/* Decode attention with the step's cache append folded in ([aitalk]     */
/* step 3: each new token's K/V goes into the next slot of the sequence's */
/* last block; step 2: the attention then reads that block through the   */
/* table).  For each sequence s with L = context_lens[s] > 0, the K/V    */
/* rows of the token at position L - 1 are first written from            */
/* k_new[s] / v_new[s] into slot (L-1) % block_size of block              */
/* block_tables[s][(L-1) / block_size] (skipped, and PKV_DEV_BAD_BLOCK_ID */
/* set, if that id is outside [0, num_blocks); a length outside          */
/* [0, max_context_len] writes nothing and sets PKV_DEV_BAD_LENGTH, so a */
/* max_context_len below the true lengths never overwrites a cached      */
/* token), then out is computed exactly as by                            */
/* paged_attention_decode.  Pools and out afterwards equal those of      */
/* paged_kv_append with that slot mapping followed by                    */
/* paged_attention_decode, bit for bit.  When num_seqs is at most the    */
/* decode workgroups per kv head (paged_attention_workgroups_per_head),   */
/* the decode kernel writes the rows itself, one launch fewer; otherwise  */
/* a small append kernel runs first on the same stream.                  */
/*                                                                        */
/* k_new, v_new  : device [num_seqs][num_kv_heads][head_dim], dtype dt,   */
/*                 16-byte aligned, not null when num_seqs > 0            */
/* k_cache, v_cache : written (one slot per sequence) and read            */
/* The block holding position L - 1 must belong to sequence s alone      */
/* (the block manager's append_slots and stage_step guarantee this by    */
/* copy-on-write); every other argument, the workspace and the errors    */
/* are as for paged_attention_decode.                                    */
int32_t paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype dt, uint32_t flags, void* stream);

/* paged_attention_decode_append without a caller workspace, for callers */
/* that cannot allocate device memory (code under HIP graph capture,      */
/* serving loops that forbid allocation): the call allocates nothing and  */
/* uses a scratch array built into the library instead, 32 MiB per GPU,   */
/* held by every GPU the library runs on until the process ends.  That is */
/* enough for the default partition_size = 0 on every supported shape up */
/* to several thousand sequences; a request whose workspace              */
/* (paged_attention_workspace_bytes at the device's occupancy) exceeds it */
/* fails with PKV_ERR_CAPACITY before any launch.  Every call on one GPU  */
/* shares that GPU's array (no content carries over between calls: each */
/* call writes what it reads), so calls that overlap on one GPU, e.g. on */
/* two streams, race; order them on one stream.  Arguments, results and  */
/* other errors are those of paged_attention_decode_append.               */
int32_t paged_attention_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_cache, void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t max_blocks_per_seq,
                                              int32_t max_context_len, float scale, int32_t partition_size,
                                              pkv_dtype dt, uint32_t flags, void* stream);

/* Workgroups per kv head that paged_attention_decode uses for these     */
/* arguments on the current device, or a negative status.                 */
int32_t paged_attention_workgroups_per_head(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_context_len, int32_t partition_size,
                                            pkv_dtype dt);

/* Fixed charge per sequence, in blocks, in the decode kernel's split of  */
/* a kv head's work ("PagedAttention" (robocikowo.com), Komponenty: the    */
/* kernel walks each sequence's block table): the blocks of all sequences */
/* form one list in which every non-empty sequence also counts this many  */
/* blocks for its fixed work (table read, query load, first K/V round     */
/* trip, cross-wave merge), and each of the W workgroups of the head      */
/* (paged_attention_workgroups_per_head) takes an equal contiguous range  */
/* of the list's C positions, [k C / W, (k+1) C / W).  block_size is 16   */
/* or 32; returns a negative status otherwise.                            */
int32_t paged_attention_segment_cost(int32_t block_size);

/* Workspace bytes paged_attention_decode needs for these arguments on    */
/* the current device (0 only when num_seqs == 0).  Returns 0 and sets    */
/* the last error for invalid arguments.                                   */
size_t paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                       int32_t partition_size);

/* Chunked-prefill attention ([aitalk] the part on the two independent    */
/* problems: a prompt's K/V are computed in the prefill phase; the part   */
/* on prefix caching: the prefill of prefixes already seen is skipped, so */
/* the rest of a prompt attends over cached blocks; step 2: the cache is  */
/* read through the block table).                                         */
/*                                                                        */
/* Sequence s owns query rows query_start[s] .. query_start[s+1]-1: its C */
/* newest tokens, whose K/V are already in the cache (paged_kv_append),   */
/* at positions L-C .. L-1 with L = context_lens[s] >= C.  The row of     */
/* position p and query head h (kv head g = h / G) is                     */
/*   out[row][h] = sum_{t<=p} softmax_t(scale * <q[row][h], K_t[g]>) V_t[g] */
/* i.e. causal attention; one-token chunks give the decode result.        */
/* Scores, softmax and the weighted sum run in fp32 on the matrix cores   */
/* (bf16 operands: the probabilities enter the value product rounded to   */
/* bf16); the output is rounded to nearest-even.                          */
/*                                                                        */
/* out, q        : device [num_tokens][num_q_heads][head_dim], bf16 only  */
/*                 (PKV_ERR_UNSUPPORTED otherwise); rows of a sequence    */
/*                 are contiguous, sequences in order                     */
/* query_start   : device int32 [num_seqs + 1], rising from 0 to          */
/*                 num_tokens; every chunk length <= max_query_len        */
/* max_query_len : host bound on the chunk lengths (sizes the launch)     */
/* block_tables, context_lens, pools: as for paged_attention_decode       */
/* scale         : > 0 (usually 1/sqrt(head_dim))                         */
/* Query group sizes up to 256 are supported.  One launch holds at most  */
/* 2^23 - 1 workgroups: num_seqs * num_kv_heads (rounded up to a multiple */
/* of 8) times ceil(max_query_len * G / 256) query tiles; larger calls    */
/* return PKV_ERR_INVALID_ARG.  No workspace; the kernel                  */
/* clamps lengths, offsets and block ids to the given sizes, so bad       */
/* device values give wrong rows, never accesses outside the buffers.    */
int32_t paged_attention_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_query_len, float scale, pkv_dtype dt, void* stream);

/* ------------------------------------------------------------------ */
/* Host block manager ([pl] Komponenty: block table, block manager with a */
/* free pool, reference counting + copy-on-write; [aitalk] steps 1-4;     */
/* [sheet] Pourquoi c'est important: pages allocated on demand and freed  */
/* one by one; [gloss] Définition: unused blocks recycled at once).      */
/*                                                                        */
/* Policy (deterministic; the pages leave it open):                       */
/*   - free pool = stack; initial_free_order[0] is handed out first;      */
/*     released blocks go on top and are reused first; a released         */
/*     sequence returns its blocks in logical order 0..n-1.               */
/*   - appending a token at length L: if L % block_size == 0 a fresh      */
/*     block is appended to the table; otherwise, if the block holding    */
/*     slot L is shared (refcount > 1), a fresh block replaces it and the */
/*     pair (old, fresh) is reported for paged_kv_copy_blocks; the slot   */
/*     is table[L / bs] * bs + L % bs.  Sequences are processed in call   */
/*     order; the last holder of a shared block writes in place.          */
/*   - every call is atomic: on error nothing changes.                    */
/* All pointers here are host pointers.                                    */
typedef struct pkv_block_manager pkv_block_manager;

/* initial_free_order: num_blocks distinct ids (a permutation), or NULL   */
/* for 0..num_blocks-1.  *out receives the handle.                        */
int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                      pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Register an empty sequence (L = 0, salt 0).  Error if the id exists. */
int32_t pkv_bm_add_seq(pkv_block_manager* bm, int64_t seq_id);

/* ---- Prefix cache ---------------------------------------------------- */
/* Chained block digests with a tenant salt ([aitalk] the closing part on  */
/* vLLM's automatic prefix caching, and the paragraph on cache salting):   */
/* every full block whose token ids are known gets                         */
/*   digest = SHA-256(parent digest (32 bytes; zeros for the first block)  */
/*                    || salt (uint64, little-endian)                      */
/*                    || its block_size token ids (int32, little-endian))  */
/* so equal token prefixes under equal salts give equal chains.            */
/* Policy (the pages leave it open):                                       */
/*   - a block is registered under its digest when it fills, if its ids    */
/*     (given to pkv_bm_append_slots / pkv_bm_stage_step with every        */
/*     append since the sequence began) and its parent's digest are known, */
/*     and no other block holds that digest (else it is a duplicate and    */
/*     stays unregistered);                                                */
/*   - a registered block whose refcount drops to 0 keeps its digest and  */
/*     joins an eviction list, oldest first; a released sequence adds its  */
/*     registered blocks from its last block to its first;                 */
/*   - new blocks come from the free stack; only when it is empty is the  */
/*     oldest evictable block taken (its digest is forgotten).             */
/*   - a registered block is immutable: a write into it (after a fork     */
/*     inside it) always copies it first, reported as a copy pair; if the */
/*     writer was its last holder it becomes evictable after the call.    */
/*     pkv_bm_num_free counts both;                                        */
/*   - without token ids nothing registers and the policy above is the    */
/*     plain free-stack one.                                               */

/* Digest of one block (host): parent = 32 bytes or NULL for zeros;       */
/* tokens [n_tokens]; out = 32 bytes.  Lets a router compute the keys a    */
/* prompt would look up.                                                   */
int32_t pkv_block_digest(const uint8_t* parent, uint64_t salt, const int32_t* tokens, int32_t n_tokens,
                         uint8_t* out);

/* Register sequence `seq_id` for a prompt tokens[0..n_tokens): its        */
/* leading full blocks are looked up in order and each registered one is  */
/* shared (refcount + 1; taken off the eviction list at 0) until the first */
/* miss.  The sequence starts at L = *n_cached_out (a multiple of          */
/* block_size, <= n_tokens) with salt `salt`; the caller appends the rest  */
/* of the prompt with its ids.  Never allocates; error if the id exists.   */
int32_t pkv_bm_add_seq_cached(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                              uint64_t salt, int32_t* n_cached_out);

/* Prompt tokens pkv_bm_add_seq_cached would share now (>= 0), changing    */
/* nothing; negative status on error.                                      */
int32_t pkv_bm_match_prefix(const pkv_block_manager* bm, const int32_t* tokens, int32_t n_tokens, uint64_t salt);

/* Registered blocks (in use or evictable).                                */
int32_t pkv_bm_num_cached(const pkv_block_manager* bm);
/* Evictable blocks, oldest (next evicted) first; returns the count;       */
/* PKV_ERR_CAPACITY if capacity is too small.                              */
int32_t pkv_bm_evictable(const pkv_block_manager* bm, int32_t* out, int32_t capacity);
/* 1 and the 32-byte digest in out if `block` is registered, else 0.       */
int32_t pkv_bm_cached_digest(const pkv_block_manager* bm, int32_t block, uint8_t* out);

/* Register `child` sharing the first ceil(num_tokens / bs) blocks of      */
/* `parent` (refcount + 1 each), with L = num_tokens <= L(parent); it      */
/* inherits the parent's salt, known token ids and digests up to there.    */
int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child, int32_t num_tokens);

/* Reserve slots for new tokens.                                           */
/* seq_ids     : [n_seqs] distinct registered ids                          */
/* num_tokens  : [n_seqs] tokens per sequence (>= 0), or NULL for 1 each   */
/* token_ids   : the new tokens' ids, in slot order (sequence-major), or    */
/*               NULL (then the sequences' digest chains end here)          */
/* slot_mapping_out : [slot_capacity]; receives the slots, sequence-major  */
/* cow_pairs_out    : [cow_capacity][2]; receives (src, dst) block copies  */
/*                    that must run before the tokens are written          */
/* *n_slots_out, *n_cow_out : counts written (either may be NULL)          */
int32_t pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                            const int32_t* num_tokens, const int32_t* token_ids, int32_t* slot_mapping_out,
                            int32_t slot_capacity,
                            int32_t* n_slots_out, int32_t* cow_pairs_out, int32_t cow_capacity,
                            int32_t* n_cow_out);

/* Release a sequence: refcount - 1 on each block; blocks reaching 0 go  */
/* back to the free pool (registered ones to the eviction list).           */
int32_t pkv_bm_free_seq(pkv_block_manager* bm, int64_t seq_id);

/* Export block tables and lengths.                                        */
/* tables_out       : [n_seqs][max_blocks_per_seq], rows padded with -1    */
/* context_lens_out : [n_seqs] (may be NULL)                               */
/* PKV_ERR_CAPACITY if a table is wider than max_blocks_per_seq.           */
int32_t pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                            int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* context_lens_out);

/* One decode step's host side without host-to-device copies.  Reserves   */
/* one slot per sequence (as pkv_bm_append_slots with one token each),    */
/* then writes a compact record into `stage` and launches, on `stream`, a */
/* small kernel that reads the record in place (over the bus) and         */
/* updates the device buffers:                                            */
/*   slot_mapping [n_seqs], context_lens [n_seqs] (after the append),     */
/*   cow_pairs [n][2] (the copies to run before writing the tokens),      */
/*   block_tables [n_seqs][max_blocks_per_seq]: only the entries that     */
/*   changed since the last call on the same table are written (new       */
/*   blocks, copy-on-write replacements, sequences that moved rows).  The */
/*   manager tracks two device tables, so a caller may alternate two      */
/*   buffer sets (stage step k+1 into one while step k still reads the    */
/*   other, e.g. on a second stream); the first call on a table, a third  */
/*   table (it replaces the least recently used one), another width, or   */
/*   full != 0 writes every used entry.  Entries past ceil(L / bs) are    */
/*   not written.                                                          */
/* A table must only be written by this function between calls.           */
/* token_ids     : host [n_seqs], the new tokens' ids, or NULL (as in     */
/*                 pkv_bm_append_slots)                                   */
/* stage         : pinned host memory (hipHostMalloc / pinned tensor) of  */
/*                 stage_capacity int32, at least                         */
/*                 pkv_bm_stage_capacity(n_seqs, max_blocks_per_seq); the */
/*                 GPU reads it after this call returns, so it must not   */
/*                 be rewritten until that kernel has run (alternate two  */
/*                 buffers and wait on an event)                          */
/* cow_pairs     : device, room for n_seqs pairs                          */
/* *n_cow_out    : pairs written; *max_len_out: largest context length    */
/* All device buffers are int32.  Errors before the reservation leave the */
/* manager unchanged.                                                     */
int32_t pkv_bm_stage_step(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs, const int32_t* token_ids,
                          int32_t* stage,
                          int32_t stage_capacity, int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t* context_lens, int32_t* slot_mapping, int32_t* cow_pairs, int32_t cow_capacity,
                          int32_t full, int32_t* n_cow_out, int32_t* max_len_out, void* stream);

/* ---- Swap to host memory -------------------------------------------- */
/* [sheet] Mode d'échec and the glossary's Page eviction: when GPU memory */
/* runs out even with paged allocation, pages are written to CPU RAM and  */
/* read back when needed.  The host pool has the device pool's format and */
/* its own block ids 0..num_host_blocks-1; the caller owns its memory     */
/* (pinned, e.g. hipHostMalloc / pin_memory) and runs the copies with     */
/* paged_kv_swap_blocks.                                                  */
/* Policy: a host free stack (id 0 handed out first, released ids on top).*/

/* Give the manager a host pool of num_host_blocks blocks (once).          */
int32_t pkv_bm_add_host_pool(pkv_block_manager* bm, int32_t num_host_blocks);

/* Move a sequence to the host pool: each of its blocks, in logical order, */
/* gets a fresh host block; pairs_out [capacity][2] receives (GPU block,   */
/* host block) copies to run before the GPU blocks are reused, and *n_pairs_out */
/* their count.  The sequence then drops its GPU references as            */
/* pkv_bm_free_seq would (blocks shared with other sequences stay, blocks */
/* with a prefix-cache digest become evictable).  While swapped out it    */
/* cannot be appended to, forked, exported or staged (PKV_ERR_INVALID_ARG);*/
/* pkv_bm_free_seq releases its host blocks.  PKV_ERR_OUT_OF_BLOCKS if    */
/* the host pool is short; atomic.                                        */
int32_t pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t capacity,
                        int32_t* n_pairs_out);

/* Bring a swapped-out sequence back: each host block, in logical order,  */
/* gets a fresh GPU block (free stack first, then the oldest evictable    */
/* block); pairs_out receives (host block, GPU block) copies to run       */
/* before the sequence is used; the host blocks are released.  The new    */
/* blocks carry no prefix-cache digest.  Atomic.                           */
int32_t pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t capacity,
                       int32_t* n_pairs_out);

int32_t pkv_bm_num_free_host(const pkv_block_manager* bm);
/* 1 if the sequence is swapped out, 0 if not, negative on error.          */
int32_t pkv_bm_is_swapped(const pkv_block_manager* bm, int64_t seq_id);

/* Worst-case stage size (int32 count) for pkv_bm_stage_step.              */
int32_t pkv_bm_stage_capacity(int32_t n_seqs, int32_t max_blocks_per_seq);

/* Queries.  Negative status on a bad handle or id.                        */
int32_t pkv_bm_num_free(const pkv_block_manager* bm);
int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);
/* Blocks of the device pool held by more than one sequence right now     */
/* (refcount >= 2), kept up to date by every call that changes a          */
/* refcount; a nonzero count is the hint for PKV_DECODE_SHARED_BLOCKS.    */
int32_t pkv_bm_num_shared(const pkv_block_manager* bm);
int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id);
int32_t pkv_bm_num_seqs(const pkv_block_manager* bm);
/* Free pool, bottom to top (the next block handed out is last);          */
/* capacity >= pkv_bm_num_free().                                          */
int32_t pkv_bm_free_stack(const pkv_block_manager* bm, int32_t* out, int32_t capacity);

/* ---- Radix-tree prefix index ---------------------------------------- */
/* [aitalk] RadixAttention : un arbre qui n'oublie pas, and the paragraph */
/* after it: a compressed trie over token sequences; a request walks it   */
/* token by token for the longest cached prefix and reuses its K/V; paths */
/* are inserted for later requests; least recently used leaves are        */
/* evicted first, nodes that requests depend on are kept; the tree only   */
/* points at blocks of the paged allocator.                               */
/* Every node is backed by a block-manager sequence (its holder, ids       */
/* 2^62 + k in creation order) forked from the request or from the node   */
/* it splits, so the tree adds references, not blocks.  A match may end   */
/* inside a block: the request then shares that partial block and the     */
/* block manager copies it on the request's first write (copy-on-write).  */
/* Host only; the block manager must outlive the index.                    */
typedef struct pkv_radix pkv_radix;
int32_t pkv_radix_create(pkv_block_manager* bm, pkv_radix** out);
/* Frees the index and releases every holder sequence. */
void pkv_radix_destroy(pkv_radix* rx);
/* Longest cached prefix of tokens[0..n_tokens) in tokens (>= 0).          */
int32_t pkv_radix_match(const pkv_radix* rx, const int32_t* tokens, int32_t n_tokens);
/* Register request `seq_id` (a new block-manager sequence) for a prompt: */
/* it shares the longest cached prefix (*n_cached_out tokens; it forks    */
/* the deepest matched node's holder) or starts empty; the matched nodes  */
/* are locked until pkv_radix_release and stamped with the current time.  */
/* The caller appends tokens[*n_cached_out..].  Error if the id exists.   */
int32_t pkv_radix_admit(pkv_radix* rx, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                        int32_t* n_cached_out);
/* Make the first n_tokens tokens of sequence seq_id (its K/V written)     */
/* reusable: an edge that diverges part way is split there, the rest      */
/* becomes a new leaf; *n_added_out = tokens added to the tree.            */
int32_t pkv_radix_insert(pkv_radix* rx, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                         int32_t* n_added_out);
/* Unlock what pkv_radix_admit locked for seq_id (the sequence itself is  */
/* freed with pkv_bm_free_seq).                                            */
int32_t pkv_radix_release(pkv_radix* rx, int64_t seq_id);
/* Free the holders of unlocked leaves, least recently used first (ties:  */
/* the older node), until pkv_bm_num_free() >= num_free_blocks or nothing */
/* is evictable; *n_evicted_out = nodes freed.                             */
int32_t pkv_radix_evict(pkv_radix* rx, int32_t num_free_blocks, int32_t* n_evicted_out);
int32_t pkv_radix_num_nodes(const pkv_radix* rx);
/* Nodes depth-first, children by first token: holder id, depth, edge     */
/* length, lock count and time stamp; returns the count.                   */
int32_t pkv_radix_nodes(const pkv_radix* rx, int64_t* holders, int32_t* depths, int32_t* edge_lens, int32_t* locks,
                        int64_t* stamps, int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
