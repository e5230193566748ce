// paged_attn_decode: one query token per sequence, context read through the
// block table, split-K over the context plus a cross-split merge.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm", section "第六站：注意力层": decode
// attends its whole history, read from the paged cache through the block
// table; the store runs first, so the context includes the current token.
//
// gfx950 design (HBM-bound: each K/V byte is read once, ~2 flop per byte):
//  * Grid (kv_head, split, seq). kv_head is the fastest index, so the
//    work-groups of all KV heads of one token range are dispatched together
//    and sweep the same 2 KiB token rows of the cache at the same time.
//  * One work-group = 4 wavefronts on one (seq, kv_head, split of `split`
//    tokens). The G = H_q / H_kv query heads of the group are computed
//    together, so every K/V byte fetched serves all G heads from registers.
//  * A wavefront handles 16 tokens per step: 8 lane groups of 8 lanes, one
//    token per group, each lane owning 32 bytes of the 256-byte head row
//    (dims 8i..8i+7 and 64+8i..64+8i+7, so every 16-byte load instruction
//    reads 128 contiguous bytes per token). q.k uses the bf16 dot2
//    instruction, then a 3-step DPP sum inside the group.
//  * Each lane group keeps its own fp32 online-softmax state (running max in
//    the log2 domain, sum, 16 x G output accumulators); the 32 states of the
//    work-group are combined once at the end (DPP/bpermute inside the
//    wavefront, LDS across the 4 wavefronts).
//  * Loads of the next 16-token step are issued before the current step is
//    computed (two register buffers).
//  * Masked positions (past the split end) load a valid row of the same
//    split and get a score of -inf, so no stale or poisoned cache row is
//    ever multiplied into the result.
//  * A sequence with a single split writes its normalised bf16 output
//    directly; otherwise the split writes (m, l, o) partials and the merge
//    kernel combines them (log-sum-exp in the log2 domain).

#include "common.h"

namespace pkv {

namespace {

constexpr float kNegBig = -1e30f;  // running-max start: finite, so m - m_new never forms inf - inf

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7-i within 8
constexpr int kRowRor8 = 0x128;     // row_ror:8 within 16 lanes

// Sum over the 8 lanes of a lane group.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float dot2acc(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot16(const u32x4& qa, const u32x4& qb, const u32x4& ka, const u32x4& kb) {
  float s = 0.f;
  s = dot2acc(qa.x, ka.x, s);
  s = dot2acc(qa.y, ka.y, s);
  s = dot2acc(qa.z, ka.z, s);
  s = dot2acc(qa.w, ka.w, s);
  s = dot2acc(qb.x, kb.x, s);
  s = dot2acc(qb.y, kb.y, s);
  s = dot2acc(qb.z, kb.z, s);
  s = dot2acc(qb.w, kb.w, s);
  return s;
}

struct Step {
  u32x4 k[2][2];  // [token t][half]
  u32x4 v[2][2];
};

template <int G>
struct State {
  float m[G];
  float l[G];
  float o[G][16];
};

__device__ __forceinline__ void load_step(Step& st, const char* __restrict__ kc, const char* __restrict__ vc,
                                          int64_t blk, int base, int wave, int grp, int li, int t_end, int hkv,
                                          int g) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int tok = base + 16 * wave + 8 * t + grp;
    tok = tok < t_end ? tok : t_end - 1;
    const int64_t row = (blk * kBlockSize + (tok & (kBlockSize - 1))) * hkv + g;
    const char* kp = kc + row * (kHeadDim * 2) + li * 16;
    const char* vp = vc + row * (kHeadDim * 2) + li * 16;
    st.k[t][0] = *reinterpret_cast<const u32x4*>(kp);
    st.k[t][1] = *reinterpret_cast<const u32x4*>(kp + 128);
    st.v[t][0] = *reinterpret_cast<const u32x4*>(vp);
    st.v[t][1] = *reinterpret_cast<const u32x4*>(vp + 128);
  }
}

template <int G>
__device__ __forceinline__ void compute_step(State<G>& S, const Step& st, const u32x4 (&qa)[G],
                                             const u32x4 (&qb)[G], int base, int wave, int grp, int t_end,
                                             float scale_log2) {
  float s[2][G];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool valid = base + 16 * wave + 8 * t + grp < t_end;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = group8_sum(dot16(qa[h], qb[h], st.k[t][0], st.k[t][1]));
      s[t][h] = valid ? x * scale_log2 : -__builtin_inff();
    }
  }
  float vf[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4& w = st.v[t][half];
      vf[t][8 * half + 0] = bf_lo(w.x);
      vf[t][8 * half + 1] = bf_hi(w.x);
      vf[t][8 * half + 2] = bf_lo(w.y);
      vf[t][8 * half + 3] = bf_hi(w.y);
      vf[t][8 * half + 4] = bf_lo(w.z);
      vf[t][8 * half + 5] = bf_hi(w.z);
      vf[t][8 * half + 6] = bf_lo(w.w);
      vf[t][8 * half + 7] = bf_hi(w.w);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mn = fmaxf(S.m[h], fmaxf(s[0][h], s[1][h]));
    const float alpha = __builtin_amdgcn_exp2f(S.m[h] - mn);
    const float p0 = __builtin_amdgcn_exp2f(s[0][h] - mn);
    const float p1 = __builtin_amdgcn_exp2f(s[1][h] - mn);
    S.l[h] = S.l[h] * alpha + (p0 + p1);
#pragma unroll
    for (int d = 0; d < 16; ++d) S.o[h][d] = S.o[h][d] * alpha + p0 * vf[0][d] + p1 * vf[1][d];
    S.m[h] = mn;
  }
}

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables, int bt_stride,
    const int32_t* __restrict__ context_lens, int hq, int hkv, int64_t num_blocks, float scale_log2,
    int max_ctx, int split, int nsplit_max, float* __restrict__ part_o, float* __restrict__ part_ml) {
  const int g = blockIdx.x;
  const int j = blockIdx.y;
  const int b = blockIdx.z;
  int L = context_lens[b];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int nsplit = (L + split - 1) / split;
  if (j >= (nsplit > 1 ? nsplit : 1)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 3;
  const int li = lane & 7;

  u32x4 qa[G], qb[G];
  const uint16_t* qrow = q + ((int64_t)b * hq + (int64_t)g * G) * kHeadDim;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qa[h] = *reinterpret_cast<const u32x4*>(qrow + h * kHeadDim + 8 * li);
    qb[h] = *reinterpret_cast<const u32x4*>(qrow + h * kHeadDim + 64 + 8 * li);
  }

  State<G> S;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    S.m[h] = kNegBig;
    S.l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) S.o[h][d] = 0.f;
  }

  if (L > 0) {
    const int t0 = j * split;
    const int t1 = t0 + split < L ? t0 + split : L;
    const int nstep = (t1 - t0 + 63) >> 6;  // 64 tokens per work-group step
    const int32_t* bt = block_tables + (int64_t)b * bt_stride;
    // a block id outside the pool is a caller error: read block 0 instead
    // (stays inside the cache; the result is unspecified)
    auto block_of = [&](int base) -> int64_t {
      const int64_t blk = bt[base >> 8];
      return (blk >= 0 && blk < num_blocks) ? blk : 0;
    };
    Step A, B;
    load_step(A, k_cache, v_cache, block_of(t0), t0, wave, grp, li, t1, hkv, g);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      retire(qa[h]);
      retire(qb[h]);
    }
    // Loads of the next step are issued unconditionally (the last one
    // re-reads the final step, an L2 hit) so that no wait is merged across
    // a conditional load.
    const int last = t0 + (nstep - 1) * 64;
    for (int it = 0; it < nstep; it += 2) {
      const int baseA = t0 + it * 64;
      const int baseB = baseA + 64 < last ? baseA + 64 : last;
      const int baseN = baseA + 128 < last ? baseA + 128 : last;
      load_step(B, k_cache, v_cache, block_of(baseB), baseB, wave, grp, li, t1, hkv, g);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
      compute_step<G>(S, A, qa, qb, baseA, wave, grp, t1, scale_log2);
      load_step(A, k_cache, v_cache, block_of(baseN), baseN, wave, grp, li, t1, hkv, g);
      __builtin_amdgcn_sched_barrier(0);
      // unconditional so that B's loads stay ahead of compute(A); a step past
      // the split end (odd step counts only) is fully masked
      compute_step<G>(S, B, qa, qb, baseA + 64, wave, grp, it + 1 < nstep ? t1 : 0, scale_log2);
    }
  }

  // ---- combine the 8 lane groups of this wavefront ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mw = fmaxf(S.m[h], dpp<kRowRor8>(S.m[h]));
    mw = fmaxf(mw, __shfl_xor(mw, 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    const float f = __builtin_amdgcn_exp2f(S.m[h] - mw);
    float lw = S.l[h] * f;
    lw += dpp<kRowRor8>(lw);
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    S.l[h] = lw;
    S.m[h] = mw;
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      float x = S.o[h][d] * f;
      x += dpp<kRowRor8>(x);
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      S.o[h][d] = x;
    }
  }

  // ---- combine the 4 wavefronts through LDS ----
  __shared__ float lds_o[4][G][kHeadDim];
  __shared__ float lds_m[4][G];
  __shared__ float lds_l[4][G];
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        lds_o[wave][h][8 * li + d] = S.o[h][d];
        lds_o[wave][h][64 + 8 * li + d] = S.o[h][8 + d];
      }
      if (li == 0) {
        lds_m[wave][h] = S.m[h];
        lds_l[wave][h] = S.l[h];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * kHeadDim; t += 256) {
    const int h = t / kHeadDim;
    const int d = t % kHeadDim;
    float M = lds_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, lds_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(lds_m[w][h] - M);
      o += lds_o[w][h][d] * f;
      l += lds_l[w][h] * f;
    }
    const int64_t qh = (int64_t)b * hq + (int64_t)g * G + h;
    if (nsplit <= 1) {
      const float r = L > 0 ? o / l : 0.f;
      out[qh * kHeadDim + d] = (uint16_t)f32_to_bf16_bits(r);
    } else {
      const int64_t pidx = qh * nsplit_max + j;
      part_o[pidx * kHeadDim + d] = o;
      if (d == 0) {
        part_ml[pidx * 2 + 0] = M;
        part_ml[pidx * 2 + 1] = l;
      }
    }
  }
}

// One wavefront per (seq, q head): combine the splits' (m, l, o).
__global__ __launch_bounds__(64) void decode_merge_kernel(uint16_t* __restrict__ out,
                                                          const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          const int32_t* __restrict__ context_lens, int hq,
                                                          int max_ctx, int split, int nsplit_max) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = context_lens[b];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int ns = (L + split - 1) / split;
  if (ns <= 1) return;
  const int lane = threadIdx.x;
  const int64_t qh = (int64_t)b * hq + h;
  const float* ml = part_ml + qh * nsplit_max * 2;
  float M = kNegBig;
  for (int j = 0; j < ns; ++j) M = fmaxf(M, ml[2 * j]);
  float a0 = 0.f, a1 = 0.f, lsum = 0.f;
  const float* po = part_o + qh * nsplit_max * kHeadDim + 2 * lane;
  for (int j = 0; j < ns; ++j) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * j] - M);
    lsum += ml[2 * j + 1] * f;
    const float2 o = *reinterpret_cast<const float2*>(po + (int64_t)j * kHeadDim);
    a0 += o.x * f;
    a1 += o.y * f;
  }
  const float inv = 1.f / lsum;
  reinterpret_cast<uint32_t*>(out + qh * kHeadDim)[lane] = pack_bf16x2(a0 * inv, a1 * inv);
}

}  // namespace

// Tokens per split: a multiple of 64 (so a 64-token step never straddles a
// 256-token block). Longer splits for larger query groups keep the partials
// small against the K/V bytes; shorter ones when there are too few
// work-groups to fill the chip.
static int decode_split_tokens(int num_seqs, int hq, int hkv, int max_ctx) {
  const int G = hq / hkv;
  int split = G >= 4 ? 512 : 256;
  while (split > 64) {
    const int64_t wgs = (int64_t)num_seqs * hkv * ((max_ctx + split - 1) / split);
    if (wgs >= 2048) break;
    split /= 2;
  }
  return split;
}

static int decode_nsplit_max(int split, int max_ctx) {
  const int n = (max_ctx + split - 1) / split;
  return n > 1 ? n : 1;
}

}  // namespace pkv

extern "C" size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t max_context_len) {
  using namespace pkv;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != kHeadDim || max_context_len < 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  const int split = decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, max_context_len);
  const int64_t ns = decode_nsplit_max(split, max_context_len);
  const int64_t units = (int64_t)num_seqs * num_q_heads * ns;
  size_t bytes = (size_t)units * kHeadDim * 4;
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)units * 2 * 4;
  return (bytes + 255) & ~(size_t)255;
}

extern "C" pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t block_table_stride,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int64_t num_blocks, float scale, int32_t max_context_len, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (num_seqs < 0 || num_blocks < 0 || max_context_len < 0 || block_table_stride < 0)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: negative size");
  if (head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: head_dim %d (128 only)", head_dim);
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: block_size %d (256 only)", block_size);
  if (num_kv_heads < 1 || num_kv_heads > 64 || num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: head counts %d/%d unsupported", num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: %d query heads per KV head (1, 2, 4 or 8)", G);
  if (!(scale > 0.f) || !__builtin_isfinite(scale))
    return fail(PKV_ERR_INVALID, "paged_attn_decode: scale must be finite and > 0");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: q, out and caches must be 16-byte aligned");
  const int64_t need_bt = (max_context_len + kBlockSize - 1) / kBlockSize;
  if (block_table_stride < need_bt)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: block_table_stride %d < %lld blocks of max_context_len",
                block_table_stride, (long long)need_bt);
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: more than 65535 sequences");
  const int split = decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, max_context_len);
  const int nsplit_max = decode_nsplit_max(split, max_context_len);
  const size_t ws = paged_attn_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len);
  if (nsplit_max > 1 && (!workspace || workspace_bytes < ws))
    return fail(PKV_ERR_WORKSPACE, "paged_attn_decode: workspace of %zu bytes needed, got %zu", ws, workspace_bytes);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: workspace must be 256-byte aligned");
  if (nsplit_max > 65535) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: context too long");

  const int64_t units = (int64_t)num_seqs * num_q_heads * nsplit_max;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                        ((units * kHeadDim * 4 + 255) & ~(int64_t)255))
                             : nullptr;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid(num_kv_heads, nsplit_max, num_seqs);
  uint16_t* o = static_cast<uint16_t*>(out);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
#define PKV_DECODE_LAUNCH(GG)                                                                                   \
  hipLaunchKernelGGL(decode_split_kernel<GG>, grid, dim3(256), 0, s, o, qq, kc, vc, block_tables,               \
                     block_table_stride, context_lens, num_q_heads, num_kv_heads, num_blocks, scale_log2,      \
                     max_context_len, split, nsplit_max, part_o, part_ml)
  switch (G) {
    case 1: PKV_DECODE_LAUNCH(1); break;
    case 2: PKV_DECODE_LAUNCH(2); break;
    case 4: PKV_DECODE_LAUNCH(4); break;
    default: PKV_DECODE_LAUNCH(8); break;
  }
#undef PKV_DECODE_LAUNCH
  pkv_status st = check_launch("paged_attn_decode (split)");
  if (st != PKV_OK) return st;
  if (nsplit_max > 1) {
    hipLaunchKernelGGL(decode_merge_kernel, dim3(num_q_heads, num_seqs), dim3(64), 0, s, o, part_o, part_ml,
                       context_lens, num_q_heads, max_context_len, split, nsplit_max);
    return check_launch("paged_attn_decode (merge)");
  }
  return ok();
}
