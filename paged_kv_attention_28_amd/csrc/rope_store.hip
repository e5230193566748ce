// rope_kv_store: rotary position embedding of q and k fused with the KV store.
//
// P2 = "读 Nano-vLLM 源码：一个极简 LLM 推理引擎是如何工作的": the attention
// layer rotates q and k by their positions and then writes K and V to the
// cache blocks. P1 = "13. 读一个最小推理引擎：nano-vllm", "第六站：注意力层":
// the store copies each token's rows to row `slot` of the cache and skips
// slot -1. Fusing the two removes the round trip of the rotated K through
// memory: K is read once, rotated in registers and written to the cache.
//
// Rotation ("rotate half", the convention of the model family of the
// workload shapes): element i of a head pairs with element i + D/2 and the
// pair turns by pos * theta^(-2i/D); cos and sin come from a table
// (pkv_rope_cos_sin) indexed by position.
//
// Layout of the work: one wavefront per token. Lane l owns head l / 8 and
// the 8-element chunks j = l % 8 and j + 8 of that head, i.e. elements
// 8j .. 8j+7 and 64+8j .. 64+8j+7, which are exactly the two halves of 8
// rotation pairs; every load and store is 16 bytes per lane, and the 8 lanes
// of a head cover its 256-byte row. Query heads beyond 8 are handled in
// further rounds of the same lanes.

#include "common.h"

namespace pkv {

namespace {

__device__ __forceinline__ float bf_at(const u32x4& v, int i) {
  const uint32_t w = v[i >> 1];
  return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// rotate the pairs (lo[i], hi[i]) of one lane by the angles whose cos / sin are c[i] / s[i]
__device__ __forceinline__ void rotate(u32x4& lo, u32x4& hi, const float (&c)[8], const float (&s)[8]) {
  u32x4 nlo, nhi;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a[2], b[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * k + e;
      const float x1 = bf_at(lo, i), x2 = bf_at(hi, i);
      a[e] = __builtin_fmaf(x1, c[i], -(x2 * s[i]));
      b[e] = __builtin_fmaf(x2, c[i], x1 * s[i]);
    }
    nlo[k] = pack_bf16x2(a[0], a[1]);
    nhi[k] = pack_bf16x2(b[0], b[1]);
  }
  lo = nlo;
  hi = nhi;
}

template <int HKV>
__global__ __launch_bounds__(256) void rope_store_kernel(uint16_t* __restrict__ q, int64_t q_stride,
                                                         const uint16_t* __restrict__ key, int64_t key_stride,
                                                         const uint16_t* __restrict__ value, int64_t value_stride,
                                                         const int32_t* __restrict__ positions,
                                                         const float* __restrict__ cos_sin, int max_pos,
                                                         char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                         const int32_t* __restrict__ slots, int64_t num_tokens,
                                                         int hq, int64_t num_slots) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 3;
  const int j = lane & 7;
  int pos = positions[t];
  pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);  // caller error: stay inside the table
  const float* cs = cos_sin + (int64_t)pos * kHeadDim + 8 * j;
  float c[8], s[8];
  {
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + kHeadDim / 2);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + kHeadDim / 2 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = c0[i];
      c[4 + i] = c1[i];
      s[i] = s0[i];
      s[4 + i] = s1[i];
    }
  }
  // K and V first (the cache store), then the query heads
  const int slot = __builtin_amdgcn_readfirstlane(slots[t]);
  if (slot >= 0 && slot < num_slots && h < HKV) {
    const uint16_t* kp = key + t * key_stride + h * kHeadDim + 8 * j;
    const uint16_t* vp = value + t * value_stride + h * kHeadDim + 8 * j;
    u32x4 klo = *reinterpret_cast<const u32x4*>(kp);
    u32x4 khi = *reinterpret_cast<const u32x4*>(kp + kHeadDim / 2);
    const u32x4 vlo = *reinterpret_cast<const u32x4*>(vp);
    const u32x4 vhi = *reinterpret_cast<const u32x4*>(vp + kHeadDim / 2);
    rotate(klo, khi, c, s);
    const int64_t row = (int64_t)slot * HKV * kHeadDim * 2 + (int64_t)h * kHeadDim * 2 + 16 * j;
    *reinterpret_cast<u32x4*>(k_cache + row) = klo;
    *reinterpret_cast<u32x4*>(k_cache + row + kHeadDim) = khi;
    *reinterpret_cast<u32x4*>(v_cache + row) = vlo;
    *reinterpret_cast<u32x4*>(v_cache + row + kHeadDim) = vhi;
  }
  for (int hh = h; hh < hq; hh += 8) {
    uint16_t* qp = q + t * q_stride + hh * kHeadDim + 8 * j;
    u32x4 lo = *reinterpret_cast<const u32x4*>(qp);
    u32x4 hi = *reinterpret_cast<const u32x4*>(qp + kHeadDim / 2);
    rotate(lo, hi, c, s);
    *reinterpret_cast<u32x4*>(qp) = lo;
    *reinterpret_cast<u32x4*>(qp + kHeadDim / 2) = hi;
  }
}

}  // namespace

}  // namespace pkv

extern "C" pkv_status pkv_rope_cos_sin(float* out, int32_t max_position, int32_t head_dim, double theta) {
  using pkv::fail;
  if (!out || max_position < 1 || head_dim < 2 || head_dim % 2)
    return fail(PKV_ERR_INVALID, "pkv_rope_cos_sin: need out, max_position >= 1 and an even head_dim");
  if (!(theta > 1.0) || !__builtin_isfinite(theta)) return fail(PKV_ERR_INVALID, "pkv_rope_cos_sin: theta > 1");
  const int half = head_dim / 2;
  for (int32_t p = 0; p < max_position; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * __builtin_pow(theta, -2.0 * i / head_dim);
      out[(int64_t)p * head_dim + i] = (float)__builtin_cos(a);
      out[(int64_t)p * head_dim + half + i] = (float)__builtin_sin(a);
    }
  return pkv::ok();
}

extern "C" pkv_status rope_kv_store(void* q, int64_t q_stride, const void* key, int64_t key_stride,
                                    const void* value, int64_t value_stride, const int32_t* positions,
                                    const float* cos_sin, int32_t max_position, void* k_cache, void* v_cache,
                                    const int32_t* slot_mapping, int64_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                    void* stream) {
  using namespace pkv;
  if (num_tokens < 0 || num_blocks < 0 || max_position < 1)
    return fail(PKV_ERR_INVALID, "rope_kv_store: negative size or max_position < 1");
  if (head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: head_dim %d (128 only)", head_dim);
  if (block_size != kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: block_size %d (256 only)", block_size);
  if (num_kv_heads != 1 && num_kv_heads != 2 && num_kv_heads != 4 && num_kv_heads != 8)
    return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: num_kv_heads %d (1, 2, 4 or 8)", num_kv_heads);
  if (num_q_heads < 1 || num_q_heads > 64)
    return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: num_q_heads %d (1 .. 64)", num_q_heads);
  if (q_stride < (int64_t)num_q_heads * kHeadDim || key_stride < (int64_t)num_kv_heads * kHeadDim ||
      value_stride < (int64_t)num_kv_heads * kHeadDim)
    return fail(PKV_ERR_INVALID, "rope_kv_store: a token stride is smaller than its row");
  if ((q_stride | key_stride | value_stride) & 7)
    return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: token strides must be multiples of 8 elements");
  if (num_tokens == 0) return ok();
  if (!q || !key || !value || !positions || !cos_sin || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "rope_kv_store: null pointer");
  if (!aligned16(q) || !aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(cos_sin))
    return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: q, key, value, caches and the table must be 16-byte aligned");
  const int64_t blocks = (num_tokens + 3) / 4;
  if (blocks > 0x7FFFFFFF) return fail(PKV_ERR_UNSUPPORTED, "rope_kv_store: too many tokens");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* qq = static_cast<uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(key);
  const uint16_t* vv = static_cast<const uint16_t*>(value);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  const int64_t num_slots = num_blocks * kBlockSize;
#define PKV_ROPE_LAUNCH(H)                                                                                    \
  hipLaunchKernelGGL(rope_store_kernel<H>, dim3((unsigned)blocks), dim3(256), 0, s, qq, q_stride, kk,         \
                     key_stride, vv, value_stride, positions, cos_sin, max_position, kc, vc, slot_mapping,     \
                     num_tokens, num_q_heads, num_slots)
  switch (num_kv_heads) {
    case 1: PKV_ROPE_LAUNCH(1); break;
    case 2: PKV_ROPE_LAUNCH(2); break;
    case 4: PKV_ROPE_LAUNCH(4); break;
    default: PKV_ROPE_LAUNCH(8); break;
  }
#undef PKV_ROPE_LAUNCH
  return check_launch("rope_kv_store");
}
