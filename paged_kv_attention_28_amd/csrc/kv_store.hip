// kv_store: scatter K/V token rows into the paged caches (bit copy).
//
// P1 = "13. 读一个最小推理引擎：nano-vllm", section "第六站：注意力层": every
// token's K and V rows are written to cache row slot_mapping[i] before
// attention; slot -1 marks a padding row and is skipped.
//
// gfx950 mapping: one 64-lane wavefront moves one token. A token row is
// num_kv_heads * 128 bf16 = num_kv_heads * 256 bytes, i.e. num_kv_heads * 16
// chunks of 16 bytes; lane i moves chunks i, i + 64, ... of K and of V, so
// each load/store instruction covers 1 KiB of contiguous row (fully
// coalesced 16-byte accesses). All loads of a lane are issued before its
// stores. The slot is read once per wave (scalar) and checked against the
// pool, so no slot can send a store outside the cache.

#include "common.h"

namespace pkv {

template <int CPL>  // 16-byte chunks per lane per row
__global__ __launch_bounds__(256) void kv_store_kernel(const char* __restrict__ key, int64_t key_stride_b,
                                                       const char* __restrict__ value, int64_t value_stride_b,
                                                       char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slots, int64_t num_tokens,
                                                       int64_t num_slots, int chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (tok >= num_tokens) return;
  const int32_t slot = __builtin_amdgcn_readfirstlane(slots[tok]);
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const u32x4* ks = reinterpret_cast<const u32x4*>(key + tok * key_stride_b);
  const u32x4* vs = reinterpret_cast<const u32x4*>(value + tok * value_stride_b);
  u32x4* kd = reinterpret_cast<u32x4*>(k_cache + (int64_t)slot * chunks * 16);
  u32x4* vd = reinterpret_cast<u32x4*>(v_cache + (int64_t)slot * chunks * 16);
  u32x4 kr[CPL], vr[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int i = lane + 64 * c;
    if (i < chunks) {
      kr[c] = ks[i];
      vr[c] = vs[i];
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int i = lane + 64 * c;
    if (i < chunks) {
      kd[i] = kr[c];
      vd[i] = vr[c];
    }
  }
}

}  // namespace pkv

extern "C" pkv_status kv_store(const void* key, int64_t key_token_stride, const void* value,
                               int64_t value_token_stride, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks, void* stream) {
  using namespace pkv;
  if (num_tokens < 0 || num_blocks < 0) return fail(PKV_ERR_INVALID, "kv_store: negative count");
  if (head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "kv_store: head_dim %d unsupported (128 only)", head_dim);
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "kv_store: block_size %d unsupported (256 only)", block_size);
  if (num_kv_heads < 1 || num_kv_heads > 16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_store: num_kv_heads %d outside 1..16", num_kv_heads);
  if (key_token_stride < 0 || value_token_stride < 0)
    return fail(PKV_ERR_INVALID, "kv_store: negative token stride");
  if (num_tokens == 0 || num_blocks == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return fail(PKV_ERR_INVALID, "kv_store: null pointer");
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (key_token_stride < row || value_token_stride < row)
    return fail(PKV_ERR_INVALID, "kv_store: token stride smaller than a row (%lld elements)", (long long)row);
  if ((key_token_stride * 2) % 16 || (value_token_stride * 2) % 16 || !aligned16(key) || !aligned16(value) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_UNSUPPORTED, "kv_store: pointers and token strides must be 16-byte aligned");
  if (num_blocks > INT64_MAX / block_size) return fail(PKV_ERR_INVALID, "kv_store: num_blocks too large");
  const int chunks = num_kv_heads * 16;
  const int cpl = (chunks + 63) / 64;
  const int64_t grid = (num_tokens + 3) / 4;
  if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "kv_store: too many tokens");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t slots = num_blocks * block_size;
  const char* k = static_cast<const char*>(key);
  const char* v = static_cast<const char*>(value);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  switch (cpl) {
    case 1:
      hipLaunchKernelGGL(kv_store_kernel<1>, dim3((uint32_t)grid), dim3(256), 0, s, k, key_token_stride * 2, v,
                         value_token_stride * 2, kc, vc, slot_mapping, num_tokens, slots, chunks);
      break;
    case 2:
      hipLaunchKernelGGL(kv_store_kernel<2>, dim3((uint32_t)grid), dim3(256), 0, s, k, key_token_stride * 2, v,
                         value_token_stride * 2, kc, vc, slot_mapping, num_tokens, slots, chunks);
      break;
    case 3:
      hipLaunchKernelGGL(kv_store_kernel<3>, dim3((uint32_t)grid), dim3(256), 0, s, k, key_token_stride * 2, v,
                         value_token_stride * 2, kc, vc, slot_mapping, num_tokens, slots, chunks);
      break;
    default:
      hipLaunchKernelGGL(kv_store_kernel<4>, dim3((uint32_t)grid), dim3(256), 0, s, k, key_token_stride * 2, v,
                         value_token_stride * 2, kc, vc, slot_mapping, num_tokens, slots, chunks);
      break;
  }
  return check_launch("kv_store");
}
