/*
 * pkv.h — C ABI of libpkv.so: paged KV-cache store and paged attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Page references:
 *   P1 = "13. 读一个最小推理引擎：nano-vllm"
 *   P2 = "读 Nano-vLLM 源码：一个极简 LLM 推理引擎是如何工作的"
 *
 * One attention layer owns two caches, K and V, each a preallocated bf16
 * tensor [num_blocks, block_size = 256, num_kv_heads, head_dim = 128]
 * (P1, "第五站：执行准备与 KV 容量": the cache is allocated once and never
 * reallocated; block size 256, P1 "第二站：一个请求的状态"). Row `slot` of the
 * flattened cache holds one token's K (or V) for all KV heads; byte offsets
 * are computed in 64 bits.
 *
 * Conventions for every call:
 *   - Pointers named "device" are caller-owned device memory (allocated by
 *     any means, e.g. torch); "host" pointers are ordinary host memory. The
 *     library never allocates or frees device memory and never synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream); kernels are
 *     enqueued on it and may still be running when the call returns.
 *   - bf16 tensors are raw 16-bit bf16 bit patterns; integer metadata is int32.
 *   - Errors are detected on the host before anything is launched. A call
 *     returns PKV_OK or an error code and then pkv_last_error() (thread-local)
 *     describes the failure. Nothing is launched on a non-OK return, except
 *     PKV_ERR_HIP, which reports a failed launch.
 *   - Device-side contents (slot values, block ids, lengths) are the caller's
 *     contract and are not checked on the host; kernels never read or write
 *     outside the cache for a slot or block id outside the pool (such rows
 *     are skipped / read as masked), but results for such inputs are
 *     unspecified.
 *   - A call with zero work returns PKV_OK without launching.
 *   - Global state: the thread-local error message, a mutex-guarded,
 *     per-device cache of the decode kernel's resident work-group count, and
 *     the scratch array of paged_attn_decode_noalloc (one per GPU).
 *     Calls from different threads on different streams are independent; a
 *     scheduler handle (pkv_sched) belongs to one thread at a time.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,     /* bad argument: null pointer, negative count, bad lengths */
  PKV_ERR_UNSUPPORTED = 2, /* valid but not supported: head_dim != 128, block_size != 256, alignment */
  PKV_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  PKV_ERR_WORKSPACE = 4    /* workspace missing or smaller than the size query returned */
};

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* ABI revision of this header; bumped on any signature change. */
int32_t pkv_abi_version(void);
#define PKV_ABI_VERSION 10

/*
 * pkv_prepare_step — per-step attention metadata, built on the host.
 *
 * P1, "第五站：执行准备与 KV 容量": the step preparation turns the scheduled
 * sequences into the model's inputs, chiefly slot_mapping, one cache row per
 * token computed this step: slot = block_table[pos / block_size] * block_size
 * + pos % block_size. P1, "第二站：一个请求的状态": the tokens computed are those
 * from num_cached onward (prefix hits, chunk continuations and decode alike).
 * P1, "第五站" (CUDA Graph paragraph): padding rows of a replayed decode batch
 * carry slot -1.
 *
 * Inputs (host):
 *   num_seqs            real sequences, >= 0
 *   seq_lens[s]         len(seq) including this step's tokens, >= 1
 *   num_cached[s]       tokens already in the cache, 0 <= num_cached < seq_len
 *   block_table_data    concatenated physical block ids of all sequences
 *   block_table_offsets[s+1]  sequence s owns data[offsets[s] .. offsets[s+1]),
 *                       at least ceil(seq_len / block_size) ids, each >= 0
 *   num_pad             padding rows appended after the real sequences
 *                       (one token each, slot -1, context length 0)
 *   block_size          tokens per block (> 0)
 *   max_blocks_per_seq  row stride of out_block_tables (>= every table length)
 *   slot_capacity       entries available in out_slot_mapping
 * Outputs (host, caller-allocated):
 *   out_slot_mapping[T]                 T = sum(seq_len - num_cached) + num_pad
 *   out_cu_seqlens_q[num_seqs+num_pad+1] prefix sums of tokens per row
 *   out_context_lens[num_seqs+num_pad]   seq_len (0 for padding rows)
 *   out_block_tables[(num_seqs+num_pad) * max_blocks_per_seq], -1 padded
 *   out_num_tokens, out_max_q_len, out_max_context_len (may be NULL)
 * Errors: PKV_ERR_INVALID for any violated condition above or a slot that
 * does not fit in int32; outputs are then unspecified.
 */
pkv_status pkv_prepare_step(int32_t num_seqs, const int32_t* seq_lens, const int32_t* num_cached,
                            const int32_t* block_table_data, const int64_t* block_table_offsets,
                            int32_t num_pad, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t* out_slot_mapping, int64_t slot_capacity,
                            int32_t* out_cu_seqlens_q, int32_t* out_context_lens,
                            int32_t* out_block_tables, int64_t* out_num_tokens,
                            int32_t* out_max_q_len, int32_t* out_max_context_len);

/*
 * kv_store — scatter this step's K and V token rows into the paged caches.
 *
 * P1, "第六站：注意力层": before attention, for prefill and decode alike, each
 * token's K and V rows (all KV heads) are copied to row slot_mapping[i] of
 * the caches; a slot of -1 (a padding row) is skipped. The copy is bit-exact.
 *
 *   key, value       device bf16, token i's row starts at key + i * key_token_stride
 *                    elements and holds num_kv_heads * head_dim contiguous
 *                    elements (a strided view of a fused QKV buffer is fine)
 *   key/value_token_stride  in elements; the byte stride must be a multiple of 16
 *   k_cache, v_cache device bf16 [num_blocks, block_size, num_kv_heads, head_dim]
 *   slot_mapping     device int32 [num_tokens]; -1 = skip. Any slot outside
 *                    [0, num_blocks * block_size) is also skipped.
 * Two tokens must not name the same slot in one call (the winner would be
 * unspecified). All pointers 16-byte aligned.
 * Errors: INVALID (null pointer, negative count), UNSUPPORTED (head_dim !=
 * 128, block_size != 256, num_kv_heads outside 1..16, misalignment), HIP.
 */
pkv_status kv_store(const void* key, int64_t key_token_stride, const void* value,
                    int64_t value_token_stride, void* k_cache, void* v_cache,
                    const int32_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, void* stream);

/*
 * Decode attention reads, for one query token per sequence, the whole
 * context through the sequence's block table (P1, "第六站：注意力层"; the
 * store runs first, so the context includes the current token).
 *
 * paged_attn_decode_workspace_size returns the bytes of device workspace
 * paged_attn_decode needs: a small header (work split) followed by fp32
 * partial results of sequences split between wavefronts (a fixed number of
 * slots per wavefront of the persistent grid). It depends only on its
 * arguments; 0 means unsupported arguments. Its contents need no
 * initialisation; calls that overlap on different streams need different
 * workspaces.
 */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len);

/*
 * paged_attn_decode — out[s, h] = softmax_j(scale * q[s,h] . K[j, g]) V[j, g]
 * over the context positions j < context_lens[s], g = h / (num_q_heads /
 * num_kv_heads) (consecutive query heads share a KV head).
 *
 *   out              device bf16 [num_seqs, num_q_heads, head_dim] (written)
 *   q                device bf16 [num_seqs, num_q_heads, head_dim] contiguous
 *   k_cache, v_cache device bf16 caches as for kv_store
 *   block_tables     device int32 [num_seqs, block_table_stride]; entry j of
 *                    row s holds the physical block of positions
 *                    [j * 256, (j + 1) * 256)
 *   context_lens     device int32 [num_seqs]; 0 marks a padding row, whose
 *                    output is all zeros
 *   max_context_len  host upper bound on context_lens (sizes the launch); a
 *                    context longer than it is an error of the caller
 *   scale            softmax scale (1/sqrt(head_dim) for the usual attention)
 *   workspace        device memory of at least workspace_size bytes (256-byte
 *                    aligned), owned by the caller, reusable across calls on
 *                    one stream
 * Supported: head_dim 128, block_size 256, num_kv_heads in {1, 2, 4, 8},
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}, num_seqs <= 8192, and
 * num_seqs * ceil(max_context_len / 2) <= 2^31 - 1 (else
 * PKV_ERR_UNSUPPORTED).
 * Results are deterministic: the split of the work depends only on the
 * context lengths, max_context_len and the device's CU count (one
 * work-group of four wavefronts per CU, on 3/4 of the CUs for one or two
 * query heads per KV head, else on all; at least 4 two-token steps per
 * wavefront), and partial results are combined in a fixed order that
 * depends on num_seqs (up to 32 sequences: 64 interleaved classes of pieces
 * per sequence and head, combined in a fixed tree; no atomics).
 * Eight query heads per KV head run instead on the MFMA tile kernel of
 * paged_attn_prefill_varlen (the sequence's new token as its one query,
 * weights rounded to bf16 for the P.V products): one work-group per (KV head,
 * sequence), or, when num_seqs x num_kv_heads < 1536, per (KV head,
 * sequence, key chunk) with up to 16 chunks of at least 4 x 32 keys, whose
 * partials (at most about 6.5 MB) go to the workspace and are merged by a
 * second kernel in chunk order; the chunking depends only on num_seqs,
 * num_kv_heads and max_context_len. With eight KV heads, eight query heads
 * per KV head take a third kernel on calls of num_seqs >= 48 with
 * max_context_len > 1024, num_seqs >= 8 with max_context_len > 4096,
 * num_seqs >= 80 with max_context_len > 768, or num_seqs >= 128 with
 * max_context_len > 512 (and num_seqs <= 8000): stream-K over 16-token tiles, one work-group of eight
 * wavefronts per CU (one per KV head), its partials (64 query heads x 1040
 * bytes per work-group) merged by the stream-K kernel's merge; the split
 * depends only on the context lengths, max_context_len and the CU count.
 * Two or four query heads per KV head take the tile kernel for small calls
 * (num_seqs <= 4; num_seqs <= 48 with two or 80 with four query heads per
 * KV head and max_context_len <= 1024; with four also num_seqs <= 32 and
 * max_context_len <= 2048), the
 * stream-K kernel otherwise. The environment variable PKV_DECODE_FORM=tile,
 * =rowwide or =rowtile, read on every call, forces one of the forms that
 * take the shape (tests, tuning): tile or rowwide for two or four query heads
 * per KV head, tile or rowtile for eight (rowtile needs eight KV heads). The
 * forms round differently (the tile forms' weights are bf16), so their
 * outputs differ within the attention tolerance, not bit for bit.
 */
pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t block_table_stride,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, float scale, int32_t max_context_len,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_noalloc — paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same kernels and the same work split as paged_attn_decode, so the
 * results are bit-identical to that call's. The partial results live in a
 * fixed 40 MiB device array inside the library (one copy per GPU, allocated
 * when the library's code object is loaded and held until the process
 * ends); the call allocates and frees nothing. The array's device address is
 * looked up once per device, on the first call with that device current.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from several threads) race and give wrong
 * results; calls on one stream are ordered and safe. Nothing in the array
 * needs to start at zero.
 *
 * Arguments: as for paged_attn_decode, without workspace / workspace_bytes.
 * Errors: as for paged_attn_decode, plus PKV_ERR_UNSUPPORTED when the
 * launch needs more than the 40 MiB (num_q_heads x 1040 bytes, both partial
 * slots, per resident wavefront, plus 4 bytes per sequence: 32 query heads
 * fit on 1024 resident wavefronts; eight query heads per KV head take the tile form
 * described under paged_attn_decode, whose partials need at most about
 * 6.5 MB, or the row-tile kernel, 64 x 1040 bytes per CU) and PKV_ERR_HIP
 * when the array's device address cannot be found.
 */
pkv_status paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t block_table_stride,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, float scale, int32_t max_context_len, void* stream);

/*
 * paged_attn_decode_store — kv_store of the step's new token followed by
 * paged_attn_decode, in one launch (P1, "第六站：注意力层": each step stores
 * the new token's K/V before attention reads the context through the block
 * table). Results equal those two calls bit for bit: the new token, at
 * position context_lens[s] - 1, is read from key/value row s instead of the
 * cache, and the wavefront that reads it also writes it to cache row
 * slot_mapping[s]; no other position of the call reads that row.
 *
 *   key, value       device bf16 [num_seqs, num_kv_heads, head_dim]; row s
 *                    (token stride in elements, 16-byte aligned rows) is the
 *                    K/V of sequence s's new token
 *   slot_mapping     device int32 [num_seqs]; the cache row of position
 *                    context_lens[s] - 1 in sequence s's block table, or -1
 *                    (padding rows, context 0) to store nothing; a slot
 *                    outside the pool is skipped
 *   k_cache, v_cache written at the slots' rows and read elsewhere
 *   other arguments  as for paged_attn_decode (same workspace size)
 * Errors: as for paged_attn_decode, plus PKV_ERR_INVALID for null
 * key/value/slot_mapping or a token stride below a row, and
 * PKV_ERR_UNSUPPORTED for rows not 16-byte aligned. Slots that disagree with
 * the block tables are the caller's error (the attention then uses the new
 * row while the cache receives it elsewhere).
 */
pkv_status paged_attn_decode_store(void* out, const void* q, const void* key, int64_t key_token_stride,
                                   const void* value, int64_t value_token_stride,
                                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, float scale, int32_t max_context_len,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_prefill_varlen — causal attention for a batch of variable-length
 * query runs whose keys are read through block tables.
 *
 * Sequence s computes n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s] query tokens,
 * the last n_s of its context of L_s = context_lens[s] tokens, so its first
 * c_s = L_s - n_s tokens are cached (a prefix hit or an earlier chunk; P1,
 * "第二站：一个请求的状态" and "第三站：调度器"). Query i of sequence s sits at
 * position c_s + i and attends keys 0 .. c_s + i (P1, "第六站：注意力层": with
 * a prefix hit or a chunk continuation the whole context is read from the
 * paged cache). K/V of the new tokens must already be stored (kv_store).
 *
 *   out              device bf16 [total_q, num_q_heads, head_dim] (written)
 *   q                device bf16 [total_q, num_q_heads, head_dim] contiguous
 *   cu_seqlens_q     device int32 [num_seqs + 1], cu[0] = 0, non-decreasing,
 *                    cu[num_seqs] = total_q
 *   context_lens     device int32 [num_seqs], L_s >= n_s
 *   block_tables     device int32 [num_seqs, block_table_stride]
 *   max_q_len        host upper bound on n_s (sizes the launch)
 *   max_context_len  host upper bound on L_s
 *   work_items       device int32 [num_work_items, 2] written by
 *                    pkv_prefill_plan for these same cu_seqlens_q,
 *                    context_lens and head counts (then one work-group per
 *                    item), or NULL (then a (num_kv_heads, num_seqs,
 *                    ceil(max_q_len / (128 / G))) grid whose work-groups past
 *                    a sequence's last tile exit at once). 8-byte aligned.
 *                    Items naming a sequence, head or tile that does not
 *                    exist are skipped. Both launches give identical bits.
 *   num_work_items   number of items (the plan's out_num_items)
 * Supported shapes as for paged_attn_decode. Deterministic.
 */
pkv_status paged_attn_prefill_varlen(void* out, const void* q, const int32_t* cu_seqlens_q,
                                     const int32_t* context_lens, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     int32_t block_table_stride, int32_t num_seqs, int32_t total_q,
                                     int32_t max_q_len, int32_t max_context_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks, float scale,
                                     const int32_t* work_items, int32_t num_work_items,
                                     void* stream);

/*
 * paged_attn_prefill_store — kv_store of the step's new tokens followed by
 * paged_attn_prefill_varlen, in one launch (P1, "第六站：注意力层": each step
 * stores the new tokens' K/V before attention reads the context through the
 * block table). Results equal those two calls bit for bit: positions
 * c_s .. L_s - 1 of sequence s (its query tokens) are read from the step's
 * key/value rows cu_seqlens_q[s] .. cu_seqlens_q[s+1] - 1 instead of the
 * cache, and the work-group that owns a query tile also writes that tile's
 * K/V rows of its KV head to cache row slot_mapping[token]; no position of
 * the call reads a row the call writes.
 *
 *   key, value       device bf16 [total_q, num_kv_heads, head_dim]; token t's
 *                    row starts at key + t * key_token_stride elements
 *                    (16-byte aligned rows; a strided view of a fused QKV
 *                    buffer works; stride at most 2^25 elements)
 *   slot_mapping     device int32 [total_q]: the cache row of each token
 *                    (as pkv_prepare_step writes it); -1 or a slot outside
 *                    the pool stores nothing
 *   k_cache, v_cache written at the slots' rows and read elsewhere
 *   other arguments  as for paged_attn_prefill_varlen (plan or grid launch)
 * Errors: as for paged_attn_prefill_varlen, plus PKV_ERR_INVALID for null
 * key/value/slot_mapping or a token stride below a row, and
 * PKV_ERR_UNSUPPORTED for rows not 16-byte aligned or strides above 2^25.
 * Slots that disagree with the block tables are the caller's error (the
 * attention then uses the new rows while the cache receives them
 * elsewhere).
 */
pkv_status paged_attn_prefill_store(void* out, const void* q, const void* key, int64_t key_token_stride,
                                    const void* value, int64_t value_token_stride,
                                    const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                    const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                    const int32_t* block_tables, int32_t block_table_stride, int32_t num_seqs,
                                    int32_t total_q, int32_t max_q_len, int32_t max_context_len,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, float scale,
                                    const int32_t* work_items, int32_t num_work_items, void* stream);

/*
 * pkv_prefill_plan — host-side work list for paged_attn_prefill_varlen.
 *
 * Part of the host step preparation (P1, "第五站：执行准备与 KV 容量": the
 * step's cu_seqlens and context lengths are built on the host before the
 * upload). One item per (sequence s, query tile t, KV head g) with at least
 * one query token, where a tile holds 128 / G consecutive query tokens
 * (G = num_q_heads / num_kv_heads). Item = {s, (t << 8) | g}. Items are
 * sorted by the number of 64-key tiles they read, ceil((c_s + end_t) / 64)
 * with end_t the tile's last query token + 1, largest first; equal costs
 * keep the order (sequence, later tile first, KV head).
 *
 *   cu_seqlens_q, context_lens  host int32, as for paged_attn_prefill_varlen
 *   out_items        host int32 [capacity, 2], or NULL to query the count
 *   capacity         items out_items can hold
 *   out_num_items    host int64 (written): number of items
 * Errors: PKV_ERR_INVALID for a malformed batch (cu_seqlens_q[0] != 0, a
 * decreasing cu_seqlens_q, a context shorter than its query run) or
 * capacity too small; PKV_ERR_UNSUPPORTED for head counts the prefill
 * kernel does not take. Nothing is written on error except the count.
 */
pkv_status pkv_prefill_plan(int32_t num_seqs, const int32_t* cu_seqlens_q,
                            const int32_t* context_lens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t* out_items, int64_t capacity,
                            int64_t* out_num_items);

/*
 * Native scheduler and block manager (host). A token-free engine loop: each
 * step decides which sequences run and which cache blocks they own; the
 * caller turns the batch into step metadata with pkv_prepare_step (and
 * pkv_prefill_plan for a prefill step) and runs the kernels.
 *
 * P1, "第三站：调度器": prefill first, FCFS from the waiting queue within
 * max_num_seqs, the token budget and the free blocks; only the first request
 * of a step may be cut to the remaining budget (its remainder stays at the
 * head of the queue); a step with any prefill runs no decode. Otherwise every
 * running sequence advances one token and, when no block is free, the most
 * recently added running sequences are preempted (their blocks freed, their
 * requests back at the front of the queue, recomputed from position 0).
 * P1, "第四站：块管理与前缀缓存": blocks for the whole current length on first
 * scheduling, one more in decode exactly when len % block_size == 1, a FIFO
 * free queue; prefix caching (token hashing) is not part of a token-free
 * scheduler. P1, "第五站": decode batches are padded to the replay buckets
 * 1, 2, 4, 8, then multiples of 16 up to 512. P1, "第一站：主循环": a
 * completed prompt yields one token and each decode step one; a request
 * finishes after output_len tokens (so it runs output_len - 1 decode steps).
 * Freed blocks are appended in table order; within a decode step sequences
 * are extended in running order; preemptions of a decode phase that leaves
 * nothing to run are reported with the next recorded step.
 *
 * Usage: create; add requests; loop { schedule; (run the step); postprocess }
 * until schedule returns kind PKV_STEP_NONE; destroy. Not thread-safe.
 */
typedef struct pkv_sched pkv_sched;

enum { PKV_STEP_NONE = -1, PKV_STEP_DECODE = 0, PKV_STEP_PREFILL = 1 };

typedef struct {
  int32_t kind;            /* PKV_STEP_PREFILL, PKV_STEP_DECODE, or PKV_STEP_NONE when all requests finished */
  int32_t num_seqs;        /* sequences in the batch */
  int32_t num_pad;         /* decode: padding rows up to the replay bucket; prefill: 0 */
  int32_t chunked_first;   /* prefill: the first sequence was cut to the remaining token budget */
  int32_t num_preempted;   /* requests preempted since the previous recorded step */
  const int32_t* request_ids;  /* [num_seqs] ids returned by pkv_sched_add */
  const int32_t* seq_lens;     /* [num_seqs] sequence length once this step's tokens are in */
  const int32_t* num_cached;   /* [num_seqs] tokens already in the cache (the step computes the rest) */
  const int32_t* full_lens;    /* [num_seqs] prompt + generated tokens of the request */
  const int64_t* bt_offsets;   /* [num_seqs + 1] CSR offsets into bt_data */
  const int32_t* bt_data;      /* block tables, concatenated */
  const int32_t* preempted;    /* [num_preempted] request ids */
} pkv_sched_batch;

/* New scheduler over a pool of num_blocks blocks (ids 0 .. num_blocks - 1).
 * PKV_ERR_INVALID for non-positive sizes. The caller owns *out. */
pkv_status pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t max_num_seqs,
                            int32_t max_num_batched_tokens, pkv_sched** out);
pkv_status pkv_sched_destroy(pkv_sched* s);

/* Queue a request (prompt_len >= 1, output_len >= 1); *out_id (if non-NULL)
 * gets its id, consecutive from 0. Not allowed between schedule and
 * postprocess. */
pkv_status pkv_sched_add(pkv_sched* s, int32_t prompt_len, int32_t output_len, int32_t* out_id);

/* Decide the next step and describe it in *out. The arrays are owned by the
 * scheduler and stay valid until the next call on it. PKV_ERR_INVALID if the
 * previous step was not postprocessed, or if nothing can run because the
 * request at the head of the queue needs more blocks than the pool holds. */
pkv_status pkv_sched_schedule(pkv_sched* s, pkv_sched_batch* out);

/* Apply the outcome of the scheduled step: prefill sequences advance by the
 * tokens they computed (a completed prompt yields one token), decode
 * sequences by one token; finished requests free their blocks. */
pkv_status pkv_sched_postprocess(pkv_sched* s);

/* Requests not finished yet (-1 for a NULL handle). */
int32_t pkv_sched_unfinished(const pkv_sched* s);

/* Blocks in the free queue (-1 for a NULL handle). */
int32_t pkv_sched_free_blocks(const pkv_sched* s);

/*
 * Decode-step graphs. P1, "第五站：执行准备与 KV 容量" (CUDA Graph paragraph):
 * decode steps are captured once per batch bucket, largest first, and
 * replayed; at run time the smallest bucket holding the batch is chosen,
 * the inputs are copied into the static buffers and the padding rows get
 * slot -1 (P1, "其余部分": small-model decode is launch-bound, which is what
 * graphs remove). Each graph holds paged_attn_decode_store (the step's
 * store fused into the split pass, then the merge) on rows [0, bucket) of
 * the buffers below, exactly as the eager call would run it; a replay gives
 * the bits of that call, which are those of kv_store followed by
 * paged_attn_decode, on the same buffer contents. As for that call, the slot
 * of row b is the cache row of position context_lens[b] - 1.
 *
 * All buffers are caller-owned device memory that must outlive the handle;
 * their contents at creation do not matter (creation only captures, it runs
 * nothing). Before each launch the caller fills rows [0, batch) and makes
 * the rows up to the chosen bucket padding rows: slot_mapping -1,
 * context_lens 0 (their output rows are written as zeros). Context lengths
 * may be anything up to max_context_len. The workspace must be sized by
 * paged_attn_decode_workspace_size for the largest bucket.
 */
typedef struct {
  const void* key;          /* device bf16 rows [rows, num_kv_heads, head_dim], token stride key_stride elements */
  int64_t key_stride;
  const void* value;        /* device bf16, as key */
  int64_t value_stride;
  const int32_t* slot_mapping;  /* device int32 [rows] */
  void* k_cache;            /* device bf16 [num_blocks, block_size, num_kv_heads, head_dim] */
  void* v_cache;
  int64_t num_blocks;
  const void* q;            /* device bf16 [rows, num_q_heads, head_dim] contiguous */
  void* out;                /* device bf16 [rows, num_q_heads, head_dim] */
  const int32_t* block_tables;  /* device int32 [rows, block_table_stride] */
  int32_t block_table_stride;
  const int32_t* context_lens;  /* device int32 [rows] */
  void* workspace;          /* device, 256-byte aligned */
  size_t workspace_bytes;
  int32_t num_q_heads, num_kv_heads, head_dim, block_size;
  float scale;
  int32_t max_context_len;
} pkv_decode_graph_desc;

typedef struct pkv_decode_graphs pkv_decode_graphs;

/* Capture one graph per bucket (buckets: ascending, >= 1; the largest sets
 * the number of rows the buffers must hold). Errors of the underlying calls
 * (shapes, alignment, workspace) are returned as those calls return them;
 * PKV_ERR_HIP if capture or instantiation fails. The caller owns *out. */
pkv_status pkv_decode_graphs_create(const pkv_decode_graph_desc* desc, const int32_t* buckets,
                                    int32_t num_buckets, pkv_decode_graphs** out);

/* The same for a whole decode step of a model: each graph holds, in order,
 * the call of every descriptor in layers[0 .. num_layers) (one per attention
 * layer: its caches, q, out, key and value rows; the metadata buffers may be
 * shared), so one replay runs all layers' stores and attention (P1, "第五站":
 * the whole decode step is captured per bucket). pkv_decode_graphs_create
 * is this call with one layer. A shared workspace is fine: the calls of one
 * replay run one after another on the replay's stream. */
pkv_status pkv_decode_graphs_create_layers(const pkv_decode_graph_desc* layers, int32_t num_layers,
                                           const int32_t* buckets, int32_t num_buckets,
                                           pkv_decode_graphs** out);

/* Replay the smallest bucket >= batch on `stream`; *out_bucket (if non-NULL)
 * gets that bucket. PKV_ERR_INVALID if batch is outside [1, largest bucket]. */
pkv_status pkv_decode_graphs_launch(pkv_decode_graphs* g, int32_t batch, int32_t* out_bucket, void* stream);

pkv_status pkv_decode_graphs_destroy(pkv_decode_graphs* g);

/*
 * rope_kv_store — rotary position embedding of q and k fused with kv_store.
 *
 * P2, attention-layer sketch: q and k are rotated by their positions, then
 * K and V are written to the cache blocks (P1, "第六站：注意力层": row `slot`
 * of the cache, slot -1 skipped). The pages give no rotation formula; this
 * library uses the "rotate half" form: element i of a head (i < head_dim/2)
 * pairs with element i + head_dim/2 and the pair turns by the angle whose
 * cosine and sine are cos_sin[pos][i] and cos_sin[pos][head_dim/2 + i]
 * (pkv_rope_cos_sin builds that table for pos * theta^(-2i/head_dim)).
 * Arithmetic in fp32, results rounded to bf16 (nearest even).
 *
 *   q            device bf16 [num_tokens, num_q_heads, head_dim] with token
 *                stride q_stride elements; rotated in place (every row,
 *                padding rows included)
 *   key, value   device bf16 [num_tokens, num_kv_heads, head_dim] rows with
 *                token strides key_stride / value_stride elements (read only)
 *   positions    device int32 [num_tokens], 0 <= pos < max_position
 *                (values outside are clamped into the table)
 *   cos_sin      device float [max_position, head_dim]
 *   slot_mapping device int32 [num_tokens]: rotated K and V of token t go to
 *                row slot_mapping[t] of the caches; -1 (or any slot outside
 *                the pool) stores nothing
 * head_dim 128, block_size 256, num_kv_heads in {1, 2, 4, 8}, num_q_heads
 * 1..64; q, key, value, caches and table 16-byte aligned; strides multiples
 * of 8 elements. Slots must be distinct within one call.
 */
pkv_status rope_kv_store(void* q, int64_t q_stride, const void* key, int64_t key_stride, const void* value,
                         int64_t value_stride, const int32_t* positions, const float* cos_sin,
                         int32_t max_position, void* k_cache, void* v_cache, const int32_t* slot_mapping,
                         int64_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, void* stream);

/* Host: out[pos][i] = cos(pos * theta^(-2i/head_dim)), out[pos][head_dim/2 + i]
 * = the sine, for pos < max_position, i < head_dim/2; computed in double and
 * rounded to float. out is host float [max_position, head_dim]; head_dim
 * even, theta > 1. */
pkv_status pkv_rope_cos_sin(float* out, int32_t max_position, int32_t head_dim, double theta);

/*
 * sample_temperature — one token per row (P1, "它省略了什么" and "第一站：主循环":
 * temperature only, the argmax of the probabilities divided by Exp(1) noise,
 * a draw with the multinomial's distribution; temperature 0 not allowed).
 * With g = -ln E supplied by the caller, the token is the first index j of
 * the largest key fp32(fp32(logits[j] * fp32(1 / T)) + g[j]) (the log of
 * the softmax differs from logits / T by a per-row constant); every step is
 * one correctly rounded fp32 operation, so the choice can be reproduced
 * exactly off the device.
 *
 *   out_tokens    device int32 [num_rows] (written)
 *   logits        device float [num_rows, vocab], row stride logits_stride
 *   temperatures  device float [num_rows], finite and > 0 (caller contract)
 *   gumbel        device float [num_rows, vocab], row stride gumbel_stride:
 *                 -ln E for independent Exp(1) draws E (finite)
 *   workspace     device, 16-byte aligned, sample_temperature_workspace_size
 *                 bytes; no initialisation needed
 * logits and gumbel 16-byte aligned with strides multiples of 4 elements.
 * Deterministic (no atomics).
 */
size_t sample_temperature_workspace_size(int32_t num_rows, int32_t vocab);
pkv_status sample_temperature(int32_t* out_tokens, const float* logits, int64_t logits_stride,
                              const float* temperatures, const float* gumbel, int64_t gumbel_stride,
                              int32_t num_rows, int32_t vocab, void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
