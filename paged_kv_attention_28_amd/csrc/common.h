// Internal helpers shared by the libpkv sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kHeadDim = 128;    // elements per head row (256 bytes of bf16)
constexpr int kBlockSize = 256;  // tokens per cache block

// Records a formatted message for pkv_last_error() and returns `code`.
pkv_status fail(pkv_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Returns PKV_OK, or PKV_ERR_HIP with the runtime's message after a launch.
pkv_status check_launch(const char* what);

// Queries (and caches) the decode kernel's resident work-group count for a
// call with these head counts and sequence count, so that a later call made
// under stream capture finds it cached; false if the device cannot be queried.
bool decode_prepare(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs);
// Clears the thread's error message (called on every successful entry).
pkv_status ok();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The step's new K/V rows for the fused store forms (paged_attn_decode_store,
// paged_attn_prefill_store): a token's row is read from k / v (the step's
// input, `*_stride_b` bytes apart) instead of the cache and written to its
// cache row slots[token]. k == nullptr when the caller stored the rows
// beforehand (paged_attn_decode, paged_attn_prefill_varlen).
struct NewRows {
  const char* k;
  const char* v;
  int64_t k_stride_b, v_stride_b;  // bytes between tokens' (decode: sequences') rows
  const int32_t* slots;            // one slot per token (decode: per sequence)
  int64_t num_slots;               // rows in each cache
  char* k_cache;                   // the caches, writable (only the slots' rows are written)
  char* v_cache;
};

// Decode on the MFMA tile kernel of the prefill path (its query is the
// sequence's one new token, at position context_lens[s] - 1): one
// work-group per (KV head, sequence), or per (KV head, sequence, key chunk)
// with a merge when the pairs are too few to fill the GPU (partials in
// `workspace`, which must hold them; else no split). Used by
// paged_attn_decode* for eight query heads per KV head, where the row-wide
// decode kernel is bound by its vector arithmetic. Arguments as validated by
// the decode entry points; head_dim 128, block 256.
pkv_status decode_tile_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int64_t num_blocks,
                            float scale, int32_t max_context_len, void* workspace, size_t workspace_bytes,
                            void* stream, const NewRows& nr);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 bit patterns packed two per dword: low and high element as fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Makes the compiler wait here until `v` has arrived (an empty asm that reads
// it). Used once, before a loop, on registers loaded ahead of the loop, so
// that the waits the compiler places inside the loop only have to cover the
// loads issued in the loop itself.
__device__ __forceinline__ void retire(const u32x4& v) { asm volatile("" ::"v"(v)); }

}  // namespace pkv
