// sample_temperature: one token per row from temperature-scaled logits and
// caller-supplied Gumbel noise.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm" ("它省略了什么", "第一站：主循环"):
// temperature-only sampling as the argmax of the probabilities divided by
// Exp(1) noise, a draw with the multinomial's distribution. With g = -ln E
// that argmax is the argmax of l * (1 / T) + g (the log of a softmax differs
// from l / T by a per-row constant), so the kernel never forms the softmax:
//   key_j = fp32( fp32(l_j * fp32(1 / T)) + g_j ),  token = first j with the largest key.
// Each operation is one correctly rounded fp32 operation (no fused
// multiply-add), so the choice is reproducible off the device.
//
// HBM-bound: 8 bytes (logit + noise) per vocabulary entry. Pass 1 splits the
// rows over about three work-groups per CU, each thread keeping four steps of
// nontemporal 16-byte loads in flight (the rows are read once), and writes
// each chunk's best (key, index) to the workspace; pass 2 reduces a row's
// chunks in one wavefront. No atomics: the result is deterministic, and the
// first-index tie-break makes it independent of the visiting order.

#include "common.h"

#pragma clang fp contract(off)

namespace pkv {

namespace {

struct Best {
  float key;
  int idx;
};

__device__ __forceinline__ bool better(float k, int i, float bk, int bi) { return k > bk || (k == bk && i < bi); }

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float k = __shfl_xor(b.key, off);
    const int i = __shfl_xor(b.idx, off);
    if (better(k, i, b.key, b.idx)) {
      b.key = k;
      b.idx = i;
    }
  }
  return b;
}

constexpr int kThreads = 256;
// Work-groups per call. Measured on 256 x 151,936 logits: 512-768 work-groups,
// each thread with four steps of nontemporal loads in flight, read 2x faster
// than 2048 work-groups with one step in flight when the caches hold dirty
// lines (59.7 vs 119 us) and 2 % faster back to back (52.1 vs 53.0 us).
constexpr int kTargetWgs = 768;

__global__ __launch_bounds__(kThreads) void sample_chunk_kernel(const float* __restrict__ logits, int64_t lstride,
                                                                const float* __restrict__ temps,
                                                                const float* __restrict__ gumbel, int64_t gstride,
                                                                int vocab, int chunk, int splits,
                                                                float2* __restrict__ part) {
  const int row = blockIdx.y;
  const int c0 = blockIdx.x * chunk;
  const int c1 = c0 + chunk < vocab ? c0 + chunk : vocab;
  const float inv = 1.0f / temps[row];
  const float* lr = logits + (int64_t)row * lstride;
  const float* gr = gumbel + (int64_t)row * gstride;
  Best b{-__builtin_inff(), c0};
  // 16-byte loads over the 4-aligned body of the chunk (chunk is a multiple of 4)
  const int body = c0 + ((c1 - c0) & ~3);
  int j = c0 + 4 * (int)threadIdx.x;
  // four steps' loads in flight before any is used
  for (; j + 3 * 4 * kThreads < body; j += 4 * 4 * kThreads) {
    f32x4 l[4], g[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      l[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lr + j + u * 4 * kThreads));
      g[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gr + j + u * 4 * kThreads));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = j + u * 4 * kThreads + e;
        const float prod = l[u][e] * inv;
        const float k = prod + g[u][e];
        if (better(k, jj, b.key, b.idx)) {
          b.key = k;
          b.idx = jj;
        }
      }
    }
  }
  for (; j < body; j += 4 * kThreads) {
    const f32x4 l = *reinterpret_cast<const f32x4*>(lr + j);
    const f32x4 g = *reinterpret_cast<const f32x4*>(gr + j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float prod = l[e] * inv;
      const float k = prod + g[e];
      if (better(k, j + e, b.key, b.idx)) {
        b.key = k;
        b.idx = j + e;
      }
    }
  }
  for (int j = body + (int)threadIdx.x; j < c1; j += kThreads) {
    const float prod = lr[j] * inv;
    const float k = prod + gr[j];
    if (better(k, j, b.key, b.idx)) {
      b.key = k;
      b.idx = j;
    }
  }
  b = wave_best(b);
  __shared__ Best wb[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wb[threadIdx.x >> 6] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r = wb[0];
    for (int w = 1; w < kThreads / 64; ++w)
      if (better(wb[w].key, wb[w].idx, r.key, r.idx)) r = wb[w];
    part[(int64_t)row * splits + blockIdx.x] = make_float2(r.key, __int_as_float(r.idx));
  }
}

__global__ __launch_bounds__(64) void sample_reduce_kernel(const float2* __restrict__ part, int splits,
                                                           int32_t* __restrict__ out) {
  const int row = blockIdx.x;
  Best b{-__builtin_inff(), 0x7FFFFFFF};
  for (int s = threadIdx.x; s < splits; s += 64) {
    const float2 p = part[(int64_t)row * splits + s];
    if (better(p.x, __float_as_int(p.y), b.key, b.idx)) {
      b.key = p.x;
      b.idx = __float_as_int(p.y);
    }
  }
  b = wave_best(b);
  if (threadIdx.x == 0) out[row] = b.idx;
}

// chunks per row: about kTargetWgs work-groups in all (three per CU), at least 4096 entries each
int splits_for(int32_t rows, int32_t vocab, int* chunk) {
  int s = (kTargetWgs + rows - 1) / rows;
  const int max_s = (vocab + 4095) / 4096;
  s = s < 1 ? 1 : (s > max_s ? max_s : s);
  int c = (vocab + s - 1) / s;
  c = (c + 3) & ~3;
  s = (vocab + c - 1) / c;
  if (chunk) *chunk = c;
  return s;
}

}  // namespace

}  // namespace pkv

extern "C" size_t sample_temperature_workspace_size(int32_t num_rows, int32_t vocab) {
  if (num_rows <= 0 || vocab <= 0) return 0;
  const size_t b = (size_t)num_rows * pkv::splits_for(num_rows, vocab, nullptr) * sizeof(float2);
  return (b + 255) & ~(size_t)255;
}

extern "C" pkv_status sample_temperature(int32_t* out_tokens, const float* logits, int64_t logits_stride,
                                         const float* temperatures, const float* gumbel, int64_t gumbel_stride,
                                         int32_t num_rows, int32_t vocab, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  using namespace pkv;
  if (num_rows < 0 || vocab < 1) return fail(PKV_ERR_INVALID, "sample_temperature: num_rows < 0 or vocab < 1");
  if (logits_stride < vocab || gumbel_stride < vocab)
    return fail(PKV_ERR_INVALID, "sample_temperature: a row stride is smaller than the vocabulary");
  if (num_rows == 0) return ok();
  if (num_rows > 65535) return fail(PKV_ERR_UNSUPPORTED, "sample_temperature: more than 65535 rows");
  if (!out_tokens || !logits || !temperatures || !gumbel)
    return fail(PKV_ERR_INVALID, "sample_temperature: null pointer");
  if (!aligned16(logits) || !aligned16(gumbel) || (logits_stride & 3) || (gumbel_stride & 3))
    return fail(PKV_ERR_UNSUPPORTED, "sample_temperature: logits and noise must be 16-byte aligned, strides x4");
  const size_t ws = sample_temperature_workspace_size(num_rows, vocab);
  if (!workspace || workspace_bytes < ws)
    return fail(PKV_ERR_WORKSPACE, "sample_temperature: workspace of %zu bytes needed, got %zu", ws, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(PKV_ERR_UNSUPPORTED, "sample_temperature: workspace must be 16-byte aligned");
  int chunk = 0;
  const int splits = splits_for(num_rows, vocab, &chunk);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float2* part = static_cast<float2*>(workspace);
  hipLaunchKernelGGL(sample_chunk_kernel, dim3(splits, num_rows), dim3(kThreads), 0, s, logits, logits_stride,
                     temperatures, gumbel, gumbel_stride, vocab, chunk, splits, part);
  pkv_status st = check_launch("sample_temperature (chunks)");
  if (st != PKV_OK) return st;
  hipLaunchKernelGGL(sample_reduce_kernel, dim3(num_rows), dim3(64), 0, s, part, splits, out_tokens);
  return check_launch("sample_temperature (reduce)");
}
