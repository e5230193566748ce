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
// Clears the thread's error message (called on every successful entry).
pkv_status ok();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 bit patterns packed two per dword: low and high element as fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 round-to-nearest-even (NaN kept quiet), as a 16-bit pattern.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

}  // namespace pkv
