// paged_attn_decode: one query token per sequence, context read through the
// block table; a persistent stream-K kernel over all context rows, then one
// wavefront per sequence merges the sequences split between wavefronts.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm", section "第六站：注意力层": decode
// attends its whole history, read from the paged cache through the block
// table; the store runs first, so the context includes the current token.
//
// gfx950 design (HBM-bound: every K/V byte is read once, ~2 flop per byte):
//  * One wavefront reads whole token rows: a K (or V) row of one token is
//    H_kv x 256 bytes; the 8 lane groups of 8 lanes cover 2 KiB, so every
//    16-byte load instruction reads 1 KiB of contiguous cache. Lane group j
//    serves KV head j % H_kv (and, when H_kv < 8, token j / H_kv of the
//    window); each lane owns 32 bytes of the head row (dims 8i..8i+7 and
//    64+8i..64+8i+7). The G query heads of the KV head are computed from the
//    same registers.
//  * q.k uses the bf16 dot2 instruction and a 3-step DPP sum inside the lane
//    group; softmax is fp32 online softmax in the log2 domain per lane group.
//  * Work split (stream-K): the context of every sequence is cut into steps
//    of 2 windows (2 tokens for H_kv = 8). Each work-group first scans the
//    context lengths in LDS; the global step list (sequence-major) is then
//    divided evenly over all wavefronts of a persistent grid, so
//    there are no empty work-groups and no tail of unequal splits. The grid
//    is one work-group per CU (the launch reserves enough LDS for that), i.e.
//    one wavefront per SIMD, on 3/4 of the CUs for one or two query heads per
//    KV head and on all CUs for four (its heavier arithmetic gains from every
//    CU): fewer, longer ranges than the two per SIMD the registers
//    would allow, which streams faster; each wavefront takes at least 4 steps.
//    A
//    wavefront walks its range across sequence boundaries with the loads of
//    the next step always in flight (two register buffers; block-table rows
//    and the next sequence's queries are prefetched). K/V loads are
//    nontemporal: the rows are read once.
//  * A wavefront that owns a whole sequence writes the normalised bf16
//    output. A sequence cut between wavefronts leaves one fp32 (m, l, o)
//    partial per piece, in slot 0 (piece starts the wavefront's range) or
//    slot 1 (piece ends it) of that wavefront. The merge kernel (one
//    work-group per sequence, all heads at once) finds the pieces from the
//    same step arithmetic and combines them (log-sum-exp in the log2
//    domain), loading them 8 at a time with the next 8 already in flight;
//    it also writes zeros for padding rows (context 0). Batches of up to 32
//    sequences, whose sequences are cut into many pieces, use a wide merge
//    (one work-group per sequence and head, 64 piece classes). (Merging
//    inside the stream kernel would need a device-scope release per piece,
//    which writes back the whole L2 of the XCD on this GPU.)
//  * Positions past the context end load the last context row (always
//    written) and get a score of -inf: stale or poisoned cache rows never
//    enter the result.
//  * Eight query heads per KV head do eight times the arithmetic of one per
//    byte, which bounds this kernel's vector FMAs; those calls run on MFMA
//    instead: the row-tile kernel below (eight KV heads, calls that stream
//    enough) or the tile form of the prefill kernel (decode_tile_call).

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "common.h"

namespace pkv {

namespace {

constexpr float kNegBig = -1e30f;  // running-max start: finite, so m - m_new never forms inf - inf
constexpr int kWavesCap = 4096;    // persistent grid cap (partial slots are sized for it)
constexpr int kMinStepsPerWave = 4;
constexpr int kWideMergeMaxSeqs = 32;  // batches up to this size merge per (sequence, head)
constexpr int kMaxSeqs = 8192;     // LDS scan capacity
// two or four query heads per KV head: calls of up to kTileFewSeqs sequences, or of up to kTileShortSeqs
// (two query heads per KV head) or kTileShortSeqsG4 (four) sequences with max_context_len up to
// kTileShortCtx, take the tile form; with four, also calls of up to kTileMidSeqsG4 sequences with
// max_context_len up to kTileMidCtx
constexpr int kTileFewSeqs = 4;
constexpr int kTileShortSeqs = 48;
constexpr int kTileShortSeqsG4 = 80;
constexpr int kTileShortCtx = 1024;
constexpr int kTileMidSeqsG4 = 32;
constexpr int kTileMidCtx = 2048;
// eight query heads per KV head: calls of at least kRowTileSeqs sequences with max_context_len above
// kRowTileCtx, of at least kRowTileLongSeqs with max_context_len above kRowTileLongCtx, of at least
// kRowTileMidSeqs with max_context_len above kRowTileMidCtx, or of at least kRowTileManySeqs with
// max_context_len above kRowTileManyCtx take the row-tile kernel; the rest the tile form
constexpr int kRowTileSeqs = 48;
constexpr int kRowTileCtx = 1024;
constexpr int kRowTileLongSeqs = 8;
constexpr int kRowTileLongCtx = 4096;
constexpr int kRowTileMidSeqs = 80;
constexpr int kRowTileMidCtx = 768;
constexpr int kRowTileManySeqs = 128;
constexpr int kRowTileManyCtx = 512;
// LDS reserved per stream work-group: more than half a CU's 160 KiB, so each
// CU holds one work-group (one wavefront per SIMD). On the 256-sequence
// decode workload this ran 6.5 % faster than two per CU: each wavefront walks
// twice as many steps and the sequences are cut into half as many pieces.
constexpr size_t kStreamLds = 90 * 1024;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7-i within 8

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

struct Buf {
  u32x4 k[2][2];  // [window t][half]
  u32x4 v[2][2];
};

template <int G>
struct State {
  float m[G];
  float l[G];
  float o[G][16];
};

// Everything a step needs; wave-uniform.
struct Step {
  int b;                   // sequence
  int s;                   // step index inside the sequence
  int64_t row0;            // cache row of the step's first token
  int last_valid_row_off;  // context length - 1 - first token of the step (>= 0)
  bool live;               // false for a padding step past the wavefront's range (fully masked)
  int32_t slot;            // fused store: cache row of the new token on the sequence's last step, else -1
};

// The step's new K/V rows (NewRows, common.h) for the fused store
// (paged_attn_decode_store): row b of k / v is sequence b's token at position
// context_lens[b] - 1, read from there instead of the cache and written to
// cache row slots[b].

template <int HKV>
__device__ __forceinline__ void load_buf(Buf& x, const char* __restrict__ kc, const char* __restrict__ vc,
                                         const Step& st, int grp, int li, const NewRows& nr) {
  constexpr int TW = 8 / HKV;
  // wave-uniform: only a sequence's last step holds its new token
  const bool from_input = nr.k && st.last_valid_row_off < 2 * TW;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int off = t * TW + grp / HKV;
    off = off < st.last_valid_row_off ? off : st.last_valid_row_off;
    const int64_t row = (st.row0 + off) * HKV + (grp % HKV);
    const char* kp = kc + row * (kHeadDim * 2) + li * 16;
    const char* vp = vc + row * (kHeadDim * 2) + li * 16;
    if (from_input && off == st.last_valid_row_off) {  // the new token: from the step's input rows
      kp = nr.k + (int64_t)st.b * nr.k_stride_b + (grp % HKV) * (kHeadDim * 2) + li * 16;
      vp = nr.v + (int64_t)st.b * nr.v_stride_b + (grp % HKV) * (kHeadDim * 2) + li * 16;
    }
    x.k[t][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
    x.k[t][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 128));
    x.v[t][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
    x.v[t][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + 128));
  }
}

// Fused store: the wavefront whose step holds a sequence's new token writes
// that token's K/V rows (already in registers) to the cache. Only the lanes
// whose own, unclamped token is the new one store, so each row is written
// once; padding steps and slots outside the pool store nothing.
template <int HKV>
__device__ __forceinline__ void store_new_row(const Buf& x, const Step& st, const NewRows& nr, int grp, int li) {
  constexpr int TW = 8 / HKV;
  const int32_t slot = st.slot;
  if (!nr.k || !st.live || st.last_valid_row_off >= 2 * TW || slot < 0 || (int64_t)slot >= nr.num_slots) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t * TW + grp / HKV != st.last_valid_row_off) continue;
    const int64_t off = ((int64_t)slot * HKV + grp % HKV) * (kHeadDim * 2) + li * 16;
    *reinterpret_cast<u32x4*>(nr.k_cache + off) = x.k[t][0];
    *reinterpret_cast<u32x4*>(nr.k_cache + off + 128) = x.k[t][1];
    *reinterpret_cast<u32x4*>(nr.v_cache + off) = x.v[t][0];
    *reinterpret_cast<u32x4*>(nr.v_cache + off + 128) = x.v[t][1];
  }
}

template <int G, int HKV, bool LAZY>
__device__ __forceinline__ void compute_buf(State<G>& S, const Buf& x, const u32x4 (&qa)[G], const u32x4 (&qb)[G],
                                            const Step& st, int grp, float scale_log2) {
  constexpr int TW = 8 / HKV;
  float sc[2][G];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool valid = st.live && (t * TW + grp / HKV) <= st.last_valid_row_off;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float d = group8_sum(dot16(qa[h], qb[h], x.k[t][0], x.k[t][1]));
      sc[t][h] = valid ? d * scale_log2 : -__builtin_inff();
    }
  }
  float vf[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4& w = x.v[t][half];
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
  if constexpr (LAZY) {
    // Lazy rescale (four query heads per KV head over long contexts, where a step's arithmetic weighs): a
    // head's reference max moves only when a score exceeds it by more than 8 (log2 units), so the weights
    // stay <= 2^8 and the 16 output multiplies are skipped whenever no lane of the wavefront moves.
    // For four heads over short contexts (more sequence starts, where the max moves) and for one or two heads
    // (memory-bound) it measured no faster, so those keep the eager form.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(sc[0][h], sc[1][h]);
      const bool grow = mx > S.m[h] + 8.f;
      const float mn = grow ? mx : S.m[h];
      const float p0 = __builtin_amdgcn_exp2f(sc[0][h] - mn);
      const float p1 = __builtin_amdgcn_exp2f(sc[1][h] - mn);
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = __builtin_amdgcn_exp2f(S.m[h] - mn);
        S.l[h] *= alpha;
#pragma unroll
        for (int d = 0; d < 16; ++d) S.o[h][d] *= alpha;
      }
      S.l[h] += p0 + p1;
#pragma unroll
      for (int d = 0; d < 16; ++d) S.o[h][d] = S.o[h][d] + p0 * vf[0][d] + p1 * vf[1][d];
      S.m[h] = mn;
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(S.m[h], fmaxf(sc[0][h], sc[1][h]));
      const float alpha = __builtin_amdgcn_exp2f(S.m[h] - mn);
      const float p0 = __builtin_amdgcn_exp2f(sc[0][h] - mn);
      const float p1 = __builtin_amdgcn_exp2f(sc[1][h] - mn);
      S.l[h] = S.l[h] * alpha + (p0 + p1);
#pragma unroll
      for (int d = 0; d < 16; ++d) S.o[h][d] = S.o[h][d] * alpha + p0 * vf[0][d] + p1 * vf[1][d];
      S.m[h] = mn;
    }
  }
}

__device__ __forceinline__ int clamp_len(int L, int max_ctx) { return L < 0 ? 0 : (L > max_ctx ? max_ctx : L); }

// Work-group scan of per-sequence step counts into LDS: pre[b] = first global
// step of sequence b, pre[S] = total.
__device__ void scan_steps(int* pre, const int32_t* __restrict__ ctx, int S, int max_ctx, int step_tok) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int per = (S + 255) / 256;
  const int lo = tid * per;
  const int hi = lo + per < S ? lo + per : S;
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += (clamp_len(ctx[b], max_ctx) + step_tok - 1) / step_tok;
  int x = sum;  // inclusive scan inside the wavefront
  const int lane = tid & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[tid >> 6] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  int run = base + x - sum;
  for (int b = lo; b < hi; ++b) {
    pre[b] = run;
    run += (clamp_len(ctx[b], max_ctx) + step_tok - 1) / step_tok;
  }
  if (tid == 255) pre[S] = base + x;
  __syncthreads();
}

// One work-group per sequence, 16 lanes per query head (8 dims per lane):
// zeros for a padding row (context 0); for a sequence split between
// wavefronts, an online log-sum-exp combination of its pieces (partials of
// up to 4 pieces are loaded at once); nothing for a sequence written whole.
// Pieces are the wavefronts wf .. wf + npieces - 1; the first one's partial
// is in slot 1 unless the sequence starts exactly at that wavefront's range.
template <int HQ>
__global__ __launch_bounds__(HQ * 16) void decode_merge_kernel(uint16_t* __restrict__ out,
                                                               const int32_t* __restrict__ header,
                                                               const float* __restrict__ part_ml,
                                                               const float* __restrict__ part_o,
                                                               const int32_t* __restrict__ context_lens) {
  const int b = blockIdx.x;
  const int h = threadIdx.x >> 4;
  const int d0 = 8 * (threadIdx.x & 15);
  const int L = context_lens[b];
  const int P = header[0];
  const int pb = header[1 + b];
  const int nb = header[2 + b] - pb;
  u32x4* op = reinterpret_cast<u32x4*>(out + ((int64_t)b * HQ + h) * kHeadDim + d0);
  if (L <= 0 || nb <= 0) {
    *op = u32x4{0, 0, 0, 0};
    return;
  }
  const int wf = pb / P;
  const int npieces = (pb + nb - 1) / P - wf + 1;
  if (npieces == 1) return;
  float M = kNegBig, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // pieces in batches of 8; the next batch is loaded before the current one
  // is combined, so only the first batch's latency is exposed
  constexpr int kBatch = HQ >= 64 ? 4 : 8;  // 1024-thread groups have half the registers
  struct Piece {
    float m[kBatch], l[kBatch];
    f32x4 lo[kBatch], hi[kBatch];
  };
  auto load = [&](Piece& pc, int i0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + k < npieces ? i0 + k : npieces - 1;
      const int w = wf + i;
      const int slot = (i == 0 && pb != w * P) ? 1 : 0;
      const int64_t pidx = ((int64_t)w * 2 + slot) * HQ + h;
      pc.m[k] = part_ml[pidx * 2];
      pc.l[k] = part_ml[pidx * 2 + 1];
      pc.lo[k] = *reinterpret_cast<const f32x4*>(part_o + pidx * kHeadDim + d0);
      pc.hi[k] = *reinterpret_cast<const f32x4*>(part_o + pidx * kHeadDim + d0 + 4);
    }
  };
  auto combine = [&](const Piece& pc, int i0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (i0 + k >= npieces) break;
      const float mn = fmaxf(M, pc.m[k]);
      const float fa = __builtin_amdgcn_exp2f(M - mn);
      const float fb = __builtin_amdgcn_exp2f(pc.m[k] - mn);
      lsum = lsum * fa + pc.l[k] * fb;
      acc[0] = acc[0] * fa + pc.lo[k].x * fb;
      acc[1] = acc[1] * fa + pc.lo[k].y * fb;
      acc[2] = acc[2] * fa + pc.lo[k].z * fb;
      acc[3] = acc[3] * fa + pc.lo[k].w * fb;
      acc[4] = acc[4] * fa + pc.hi[k].x * fb;
      acc[5] = acc[5] * fa + pc.hi[k].y * fb;
      acc[6] = acc[6] * fa + pc.hi[k].z * fb;
      acc[7] = acc[7] * fa + pc.hi[k].w * fb;
      M = mn;
    }
  };
  Piece cur, nxt;
  load(cur, 0);
  for (int i0 = 0; i0 < npieces; i0 += kBatch) {
    const bool more = i0 + kBatch < npieces;
    if (more) load(nxt, i0 + kBatch);
    combine(cur, i0);
    if (more) cur = nxt;
  }
  const float inv = 1.f / lsum;
  *op = u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
}

// Small-batch merge: one work-group per (sequence, query head), 64 piece
// classes of 16 lanes (8 dims per lane); class c combines pieces c, c + 64,
// ... (4 loaded at once, the next 4 in flight), so a sequence of up to 64
// pieces costs one round of loads. The classes then meet in two stages: the
// four classes of a wavefront by lane exchanges (lane ^ 16, lane ^ 32), the
// sixteen wavefronts through LDS, where wavefront 0 combines four entries per
// lane group and exchanges once more. Zeros for a padding row.
template <int HQ>
__global__ __launch_bounds__(1024) void decode_merge_wide_kernel(uint16_t* __restrict__ out,
                                                                 const int32_t* __restrict__ header,
                                                                 const float* __restrict__ part_ml,
                                                                 const float* __restrict__ part_o,
                                                                 const int32_t* __restrict__ context_lens) {
  constexpr int kClasses = 64;
  constexpr int kBatch = 4;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int c = threadIdx.x >> 4;
  const int d0 = 8 * (threadIdx.x & 15);
  const int L = context_lens[b];
  const int P = header[0];
  const int pb = header[1 + b];
  const int nb = header[2 + b] - pb;
  u32x4* op = reinterpret_cast<u32x4*>(out + ((int64_t)b * HQ + h) * kHeadDim + d0);
  if (L <= 0 || nb <= 0) {
    if (c == 0) *op = u32x4{0, 0, 0, 0};
    return;
  }
  const int wf = pb / P;
  const int npieces = (pb + nb - 1) / P - wf + 1;
  if (npieces == 1) return;
  const int nsub = (npieces - c + kClasses - 1) / kClasses;
  float M = kNegBig, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto comb = [&](float m2, float l2, const float (&a2)[8]) {
    const float mn = fmaxf(M, m2);
    const float fa = __builtin_amdgcn_exp2f(M - mn);
    const float fb = __builtin_amdgcn_exp2f(m2 - mn);
    lsum = lsum * fa + l2 * fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * fa + a2[e] * fb;
    M = mn;
  };
  struct Piece {
    float m[kBatch], l[kBatch];
    f32x4 lo[kBatch], hi[kBatch];
  };
  auto load = [&](Piece& pc, int j0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = c + kClasses * (j0 + k < nsub ? j0 + k : nsub - 1);
      const int w = wf + i;
      const int slot = (i == 0 && pb != w * P) ? 1 : 0;
      const int64_t pidx = ((int64_t)w * 2 + slot) * HQ + h;
      pc.m[k] = part_ml[pidx * 2];
      pc.l[k] = part_ml[pidx * 2 + 1];
      pc.lo[k] = *reinterpret_cast<const f32x4*>(part_o + pidx * kHeadDim + d0);
      pc.hi[k] = *reinterpret_cast<const f32x4*>(part_o + pidx * kHeadDim + d0 + 4);
    }
  };
  if (nsub > 0) {
    Piece cur, nxt;
    load(cur, 0);
    for (int j0 = 0; j0 < nsub; j0 += kBatch) {
      const bool more = j0 + kBatch < nsub;
      if (more) load(nxt, j0 + kBatch);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (j0 + k >= nsub) break;
        const float a2[8] = {cur.lo[k].x, cur.lo[k].y, cur.lo[k].z, cur.lo[k].w,
                             cur.hi[k].x, cur.hi[k].y, cur.hi[k].z, cur.hi[k].w};
        comb(cur.m[k], cur.l[k], a2);
      }
      if (more) cur = nxt;
    }
  }
  auto exchange = [&]() {  // combine with lanes ^ 16 and ^ 32 (the other classes of this wavefront)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(M, off);
      const float l2 = __shfl_xor(lsum, off);
      float a2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[e], off);
      comb(m2, l2, a2);
    }
  };
  exchange();
  __shared__ float red[16][10][16];
  const int wv = threadIdx.x >> 6;
  const int ln = threadIdx.x & 63;
  if (ln < 16) {
    red[wv][0][ln] = M;
    red[wv][1][ln] = lsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wv][2 + e][ln] = acc[e];
  }
  __syncthreads();
  if (wv != 0) return;
  M = kNegBig;
  lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const int g = ln >> 4, t = ln & 15;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int src = g + 4 * k;
    float a2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a2[e] = red[src][2 + e][t];
    comb(red[src][0][t], red[src][1][t], a2);
  }
  exchange();
  if (ln >= 16) return;
  const float inv = 1.f / lsum;
  *op = u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
}

template <int G, int HKV, bool LAZY>
__global__ __launch_bounds__(256) void decode_stream_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables, int bt_stride,
    const int32_t* __restrict__ context_lens, int num_seqs, int64_t num_blocks, float scale_log2, int max_ctx,
    int32_t* __restrict__ header, float* __restrict__ part_ml, float* __restrict__ part_o, const NewRows nr) {
  constexpr int TW = 8 / HKV;       // tokens per window (one load covers TW token rows)
  constexpr int STEP_TOK = 2 * TW;  // tokens per step
  constexpr int HQ = G * HKV;
  extern __shared__ int pre[];      // [num_seqs + 1]

  scan_steps(pre, context_lens, num_seqs, max_ctx, STEP_TOK);
  const int T = pre[num_seqs];
  const int W = gridDim.x * 4;
  int P = (T + W - 1) / W;
  P = P > kMinStepsPerWave ? P : kMinStepsPerWave;
  if (blockIdx.x == 0) {  // step prefix for the merge kernel
    for (int i = threadIdx.x; i <= num_seqs; i += 256) header[1 + i] = pre[i];
    if (threadIdx.x == 0) header[0] = P;
  }

  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s0 = w * P;
  if (s0 >= T) return;
  const int s1 = s0 + P < T ? s0 + P : T;
  const int grp = lane >> 3;
  const int li = lane & 7;
  const int kvh = grp % HKV;

  // sequence holding global step s0: pre[lo] <= s0 < pre[lo + 1]
  int lo_b = 0, hi_b = num_seqs;
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (pre[mid] <= s0) lo_b = mid; else hi_b = mid;
  }
  const int b0 = __builtin_amdgcn_readfirstlane(lo_b);

  auto next_seq = [&](int b) -> int {  // next sequence with at least one step (num_seqs if none)
    int nb = b + 1;
    while (nb < num_seqs && pre[nb + 1] == pre[nb]) ++nb;
    return nb;
  };
  auto bt_row = [&](int b, uint32_t& r0, uint32_t& r1) {  // lane i: entries i and 64 + i
    const int32_t* row = block_tables + (int64_t)(b < num_seqs ? b : 0) * bt_stride;
    r0 = lane < bt_stride ? (uint32_t)row[lane] : 0u;
    r1 = 64 + lane < bt_stride ? (uint32_t)row[64 + lane] : 0u;
  };
  auto q_row = [&](int b, auto& xa, auto& xb) {
    const uint16_t* qp = q + ((int64_t)(b < num_seqs ? b : 0) * HQ + kvh * G) * kHeadDim + 8 * li;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      xa[h] = *reinterpret_cast<const u32x4*>(qp + h * kHeadDim);
      xb[h] = *reinterpret_cast<const u32x4*>(qp + h * kHeadDim + 64);
    }
  };

  // ---- load position: sequence, step, block-table rows (current and next) ----
  int ld_b = b0;
  int ld_s = s0 - pre[b0];
  int ld_L = clamp_len(context_lens[ld_b], max_ctx);
  int ld_n = pre[ld_b + 1] - pre[ld_b];
  uint32_t bt0, bt1, btn0, btn1;
  bt_row(ld_b, bt0, bt1);
  int ld_next = next_seq(ld_b);
  bt_row(ld_next, btn0, btn1);
  int ld_next_L = ld_next < num_seqs ? clamp_len(context_lens[ld_next], max_ctx) : 0;
  int ld_g = s0;  // global index of the load position

  auto make_step = [&]() -> Step {
    Step st;
    const int tok0 = ld_s * STEP_TOK;
    const int j = tok0 >> 8;
    int64_t blk;
    if (j < 64) blk = (int32_t)__builtin_amdgcn_readlane(bt0, j);
    else if (j < 128) blk = (int32_t)__builtin_amdgcn_readlane(bt1, j - 64);
    else blk = block_tables[(int64_t)ld_b * bt_stride + j];
    if (blk < 0 || blk >= num_blocks) blk = 0;  // caller error: stay inside the pool
    st.b = ld_b;
    st.s = ld_s;
    st.row0 = blk * kBlockSize + (tok0 & (kBlockSize - 1));
    st.last_valid_row_off = ld_L - 1 - tok0;
    st.live = true;
    // fused store: the slot is read when the last step is made, a step before it is used
    st.slot = (nr.k && st.last_valid_row_off < STEP_TOK) ? nr.slots[ld_b] : -1;
    return st;
  };
  auto advance_load = [&]() {
    ++ld_g;
    if (++ld_s == ld_n && ld_g < s1) {
      ld_b = ld_next;
      ld_s = 0;
      ld_L = ld_next_L;
      ld_n = pre[ld_b + 1] - pre[ld_b];
      bt0 = btn0;
      bt1 = btn1;
      ld_next = next_seq(ld_b);
      bt_row(ld_next, btn0, btn1);
      ld_next_L = ld_next < num_seqs ? clamp_len(context_lens[ld_next], max_ctx) : 0;
    }
  };
  auto padding_step = [](const Step& like) {
    Step st = like;
    st.live = false;
    return st;
  };

  // ---- compute position: queries of its sequence (and, for G <= 2, of the
  // next one, prefetched; larger groups reload at the switch to save registers)
  constexpr bool kPrefetchQ = G <= 2;
  constexpr int GN = kPrefetchQ ? G : 1;
  u32x4 qa[G], qb[G], qna[GN], qnb[GN];
  q_row(b0, qa, qb);
  if constexpr (kPrefetchQ) q_row(next_seq(b0), qna, qnb);
  State<G> S;
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      S.m[h] = kNegBig;
      S.l[h] = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) S.o[h][d] = 0.f;
    }
  };
  reset();
  int piece_first = s0;  // global index of the current piece's first step

  // After the last step of a piece (sequence end or range end): combine the
  // lane groups of each head, then write the output or a partial.
  auto finish_piece = [&](const Step& st, int gidx) {
    const int pb = pre[st.b];
    const int nb = pre[st.b + 1] - pb;
    if (HKV < 8) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int off = 8 * HKV; off < 64; off <<= 1) {
          const float mo = __shfl_xor(S.m[h], off);
          const float mn = fmaxf(S.m[h], mo);
          const float fa = __builtin_amdgcn_exp2f(S.m[h] - mn);
          const float fb = __builtin_amdgcn_exp2f(mo - mn);
          S.l[h] = S.l[h] * fa + __shfl_xor(S.l[h], off) * fb;
#pragma unroll
          for (int d = 0; d < 16; ++d) S.o[h][d] = S.o[h][d] * fa + __shfl_xor(S.o[h][d], off) * fb;
          S.m[h] = mn;
        }
      }
    }
    const bool whole = (pb / P) == ((pb + nb - 1) / P);
    if (grp < HKV) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int head = kvh * G + h;
        if (whole) {
          const float inv = 1.f / S.l[h];
          u32x4 a, c;
          a.x = pack_bf16x2(S.o[h][0] * inv, S.o[h][1] * inv);
          a.y = pack_bf16x2(S.o[h][2] * inv, S.o[h][3] * inv);
          a.z = pack_bf16x2(S.o[h][4] * inv, S.o[h][5] * inv);
          a.w = pack_bf16x2(S.o[h][6] * inv, S.o[h][7] * inv);
          c.x = pack_bf16x2(S.o[h][8] * inv, S.o[h][9] * inv);
          c.y = pack_bf16x2(S.o[h][10] * inv, S.o[h][11] * inv);
          c.z = pack_bf16x2(S.o[h][12] * inv, S.o[h][13] * inv);
          c.w = pack_bf16x2(S.o[h][14] * inv, S.o[h][15] * inv);
          uint16_t* op = out + ((int64_t)st.b * HQ + head) * kHeadDim + 8 * li;
          *reinterpret_cast<u32x4*>(op) = a;
          *reinterpret_cast<u32x4*>(op + 64) = c;
        } else {
          const int slot = (piece_first == s0) ? 0 : 1;
          const int64_t pidx = ((int64_t)w * 2 + slot) * HQ + head;
          float* po = part_o + pidx * kHeadDim + 8 * li;
          *reinterpret_cast<f32x4*>(po) = f32x4{S.o[h][0], S.o[h][1], S.o[h][2], S.o[h][3]};
          *reinterpret_cast<f32x4*>(po + 4) = f32x4{S.o[h][4], S.o[h][5], S.o[h][6], S.o[h][7]};
          *reinterpret_cast<f32x4*>(po + 64) = f32x4{S.o[h][8], S.o[h][9], S.o[h][10], S.o[h][11]};
          *reinterpret_cast<f32x4*>(po + 68) = f32x4{S.o[h][12], S.o[h][13], S.o[h][14], S.o[h][15]};
          if (li == 0) {
            part_ml[pidx * 2 + 0] = S.m[h];
            part_ml[pidx * 2 + 1] = S.l[h];
          }
        }
      }
    }
    reset();
    piece_first = gidx + 1;
    if (st.s + 1 == nb) {  // the sequence ended: move to the next one's queries
      if constexpr (kPrefetchQ) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          qa[h] = qna[h];
          qb[h] = qnb[h];
        }
        q_row(next_seq(next_seq(st.b)), qna, qnb);
      } else {
        q_row(next_seq(st.b), qa, qb);
      }
    }
  };
  auto ends_piece = [&](const Step& st, int gidx) {
    return st.s + 1 == pre[st.b + 1] - pre[st.b] || gidx + 1 == s1;
  };

  Buf A, B;
  Step sa = make_step();
  load_buf<HKV>(A, k_cache, v_cache, sa, grp, li, nr);
  advance_load();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    retire(qa[h]);
    retire(qb[h]);
  }
  for (int gi = s0; gi < s1; gi += 2) {
    // The loads of the following step are issued unconditionally (a padding
    // step past the range re-reads rows just fetched and is fully masked),
    // so they are never sunk below the compute of the current step.
    const bool hasB = gi + 1 < s1;
    const Step sb = hasB ? make_step() : padding_step(sa);
    load_buf<HKV>(B, k_cache, v_cache, sb, grp, li, nr);
    if (hasB) advance_load();
    __builtin_amdgcn_sched_barrier(0);
    compute_buf<G, HKV, LAZY>(S, A, qa, qb, sa, grp, scale_log2);
    store_new_row<HKV>(A, sa, nr, grp, li);
    if (ends_piece(sa, gi)) finish_piece(sa, gi);
    const bool hasA = gi + 2 < s1;
    const Step sn = hasA ? make_step() : padding_step(sb);
    load_buf<HKV>(A, k_cache, v_cache, sn, grp, li, nr);
    if (hasA) advance_load();
    __builtin_amdgcn_sched_barrier(0);
    compute_buf<G, HKV, LAZY>(S, B, qa, qb, sb, grp, scale_log2);
    if (hasB) store_new_row<HKV>(B, sb, nr, grp, li);
    if (hasB && ends_piece(sb, gi + 1)) finish_piece(sb, gi + 1);
    sa = sn;
  }
}

// ---------------------------------------------------------------------------
// Row-tile decode (eight query heads per KV head, eight KV heads: 64 Q /
// 8 KV): stream-K over 16-token tiles, one work-group of eight wavefronts per
// CU, wavefront g streaming KV head g.
//
// A tile is 16 consecutive tokens of one sequence (inside one cache block).
// The global tile list (sequences in order) is divided evenly over the
// work-groups. A work-group moves its tiles' whole K and V rows (2 KiB per
// token, all eight heads) into a two-stage LDS buffer with direct-to-LDS
// buffer loads (nontemporal; each wavefront moves two tokens, 1 KiB per
// instruction), one tile in flight while the previous one is computed, with
// a barrier before and after each tile's computation; wavefront g reads head
// g's 256-byte column of the rows: K in the layout of the MFMA A operand, V^T
// through the transposing LDS read. The first tile of each sequence also
// brings the sequence's eight query rows of the head group into registers.
// S^T = K_g Q^T with
// v_mfma_f32_16x16x32_bf16 (16 keys x 16 query rows, the G query heads of
// the KV head padded to 16), an online softmax per query row across the four
// lane groups that hold its 16 scores, and O^T += V_g^T P^T with
// v_mfma_f32_16x16x16_bf16, whose B operand is the weights exactly as the
// S^T accumulators hold them (lane l: keys 4 (l / 16) .. + 3 of query row
// l % 16). Sequences cut between work-groups leave fp32 (m, l, o) partials
// in the same layout as the row-wide kernel (work-group w, slot 0 for the
// piece that starts its range, slot 1 for the one that ends it), so the same
// merge kernels combine them, with tiles as the steps. The 16-byte chunks of
// row t are XOR-swizzled in LDS (by t % 16 for K, 4 t % 16 for V), which
// keeps the operand reads free of bank conflicts. Positions past the context
// load its last row (always written) and are masked.
// ---------------------------------------------------------------------------

constexpr int kRT = 16;                             // tokens per row tile
constexpr int kRTKv = 8;                            // KV heads (one wavefront each)
constexpr int kRTRow = kRTKv * kHeadDim * 2;        // 2 KiB: one token's K (or V) row
constexpr int kRTMinTiles = 2;                      // tiles per work-group at least
constexpr int kRTMaxSeqs = 8000;                    // LDS scan capacity beside the two tile stages

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
template <int N>
struct RTStage {
  static constexpr int value = N;
};
// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at their maxima; gfx9 encoding)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4k + c names row k, 4-element chunk c; lane i receives element i of the
// group's 4 x 16 block from rows 0..3.
__device__ __forceinline__ uint2 rt_read_tr16(const char* __restrict__ p) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
#pragma clang diagnostic pop
  return __builtin_bit_cast(uint2, v);
}

// Work-group scan of per-sequence tile counts (NT threads): pre[b] = first
// global tile of sequence b, pre[S] = total.
template <int NT>
__device__ void scan_units(int* pre, const int32_t* __restrict__ ctx, int S, int max_ctx, int unit) {
  __shared__ int wsum[NT / 64];
  const int tid = threadIdx.x;
  const int per = (S + NT - 1) / NT;
  const int lo = tid * per;
  const int hi = lo + per < S ? lo + per : S;
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += (clamp_len(ctx[b], max_ctx) + unit - 1) / unit;
  int x = sum;  // inclusive scan inside the wavefront
  const int lane = tid & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[tid >> 6] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  int run = base + x - sum;
  for (int b = lo; b < hi; ++b) {
    pre[b] = run;
    run += (clamp_len(ctx[b], max_ctx) + unit - 1) / unit;
  }
  if (tid == NT - 1) pre[S] = base + x;
  __syncthreads();
}

// One tile of the work-group's range: sequence, tile index inside it, first token, valid tokens, cache block.
struct RowTile {
  int b, st, tok0, nvalid;
  int blk;    // cache block (checked against the pool)
  int last;   // last tile of its sequence
  int qload;  // the wavefront starts this sequence here: its query rows come with the tile
};

constexpr int kNtAux = 2;                            // buffer-load cache policy: nontemporal
constexpr int kRTStages = 2;                         // LDS stages: one tile loading while one is computed
constexpr int kRTTileRows = kRT * kRTRow;            // 32 KiB: a tile's K (or V) rows, all eight heads
constexpr int kRTStage = 2 * kRTTileRows;            // 64 KiB: K rows, then V rows
__host__ __device__ constexpr int rt_lds_fixed(int) { return kRTStages * kRTStage; }

template <int G, bool FUSED>
__global__ __launch_bounds__(512) void decode_rowtile_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ block_tables, int bt_stride,
    const int32_t* __restrict__ context_lens, int num_seqs, int64_t num_blocks, float scale_log2, int max_ctx,
    int32_t* __restrict__ header, float* __restrict__ part_ml, float* __restrict__ part_o, const NewRows nr) {
  constexpr int HQ = G * kRTKv;
  // two stages of a tile's K and V rows (all eight heads), then the tile prefix
  extern __shared__ __attribute__((aligned(16))) char rt_lds[];
  int* pre = reinterpret_cast<int*>(rt_lds + rt_lds_fixed(G));

  scan_units<512>(pre, context_lens, num_seqs, max_ctx, kRT);
  const int T = pre[num_seqs];
  const int W = gridDim.x;
  int P = (T + W - 1) / W;
  P = P > kRTMinTiles ? P : kRTMinTiles;
  if (blockIdx.x == 0) {  // tile prefix and tiles per work-group for the merge kernel
    for (int i = threadIdx.x; i <= num_seqs; i += 512) header[1 + i] = pre[i];
    if (threadIdx.x == 0) header[0] = P;
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  }
  const int s0 = blockIdx.x * P;
  if (s0 >= T) return;
  const int s1 = s0 + P < T ? s0 + P : T;
  const int n = s1 - s0;

  const int lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // KV head of this wavefront
  const int col = lane & 15;   // query row of the MFMA tiles; key row of the K operand
  const int grp = lane >> 4;   // lane group: keys 4 grp .. 4 grp + 3 of the S^T tile
  const bool row_real = col < G;
  const uint32_t nblk32 = num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)num_blocks;

  // sequence holding global tile s0: pre[lo] <= s0 < pre[lo + 1]
  int lo_b = 0, hi_b = num_seqs;
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (pre[mid] <= s0) lo_b = mid; else hi_b = mid;
  }
  // tile metadata is wave-uniform: the sequence index goes through readfirstlane so that its context length
  // and block id are scalar loads
  auto rfl = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  auto make_tile = [&](int b, int st) -> RowTile {
    RowTile t;
    t.b = rfl(b);
    t.st = rfl(st);
    t.tok0 = t.st * kRT;
    const int L = clamp_len(context_lens[t.b], max_ctx);
    t.nvalid = L - t.tok0 < kRT ? L - t.tok0 : kRT;
    t.last = rfl(t.st + 1 == pre[t.b + 1] - pre[t.b] ? 1 : 0);
    const uint32_t blk32 = (uint32_t)block_tables[(int64_t)t.b * bt_stride + (t.tok0 >> 8)];
    t.blk = rfl(blk32 < nblk32 ? (int)blk32 : 0);  // caller error: stay inside the pool
    t.nvalid = rfl(t.nvalid);
    t.qload = t.st == 0 ? 1 : 0;
    return t;
  };
  auto next_tile = [&](const RowTile& t) -> RowTile {
    if (!t.last) return make_tile(t.b, t.st + 1);
    int nb = t.b + 1;
    while (nb < num_seqs && pre[nb + 1] == pre[nb]) ++nb;
    return make_tile(nb < num_seqs ? nb : t.b, 0);  // past the last sequence only when the range ends there
  };

  // Loads of a tile into LDS stage ST, shared by the work-group: the first tile of a sequence brings this
  // wavefront's query rows into the stage's registers first; then wavefront w moves tokens 2 w and 2 w + 1 of
  // the tile, K and V, each 2 KiB row as two 1 KiB buffer loads with the lds bit (nontemporal: the rows are
  // read once). Lane l of half hf writes the row's LDS chunk 64 hf + l, i.e. head 4 hf + l / 16, physical chunk
  // l % 16, which holds that head's logical chunk (l % 16) ^ (t % 16) of K and (l % 16) ^ (4 t % 16) of V.
  // Tokens past the context load its last row; with the fused store, the sequence's new token (its last
  // position) comes from the step's input row. (Buffer loads, not global_load_lds: the compiler treats an
  // LDS-writing global instruction like a flat access and then waits for every load in flight. Each wavefront
  // streaming its own head's 256-byte slices, two tiles in flight in registers and no barrier, ran 0-6 %
  // slower.)
  u32x4 qst[kRTStages][4];
  auto issue = [&](auto stage_c, const RowTile& t) {
    constexpr int ST = decltype(stage_c)::value;
    if (t.qload) {
      const uint16_t* qp = q + ((int64_t)t.b * HQ + g * G + (row_real ? col : 0)) * kHeadDim + 8 * grp;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qst[ST][kk] = row_real ? *reinterpret_cast<const u32x4*>(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
    }
    char* kb = rt_lds + ST * kRTStage;
    char* vb = kb + kRTTileRows;
    const int64_t row0 = (int64_t)t.blk * kBlockSize + (t.tok0 & (kBlockSize - 1));
    const bool from_input = FUSED && nr.k && t.last;
    const int t_new = t.nvalid - 1;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + row0 * kRTRow), (short)0, kRTTileRows, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + row0 * kRTRow), (short)0, kRTTileRows, 0x00020000);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int tr = 2 * g + r;
      const int te = tr < t.nvalid ? tr : t_new;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t hoff = (uint32_t)((4 * hf + grp) * (kHeadDim * 2));
        const uint32_t kc = (uint32_t)(16 * (col ^ (tr & 15)));
        const uint32_t vc = (uint32_t)(16 * (col ^ ((4 * tr) & 15)));
        lds_void_t* kd = (lds_void_t*)(kb + tr * kRTRow + 1024 * hf);
        lds_void_t* vd = (lds_void_t*)(vb + tr * kRTRow + 1024 * hf);
        if (from_input && te == t_new) {
          const __amdgpu_buffer_rsrc_t ki = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(nr.k + (int64_t)t.b * nr.k_stride_b), (short)0, kRTRow, 0x00020000);
          const __amdgpu_buffer_rsrc_t vi = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(nr.v + (int64_t)t.b * nr.v_stride_b), (short)0, kRTRow, 0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ki, kd, 16, hoff + kc, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vi, vd, 16, hoff + vc, 0, 0, 0);
        } else {
          const uint32_t roff = (uint32_t)(te * kRTRow) + hoff;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kd, 16, roff + kc, 0, 0, kNtAux);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vd, 16, roff + vc, 0, 0, kNtAux);
        }
      }
    }
#pragma clang diagnostic pop
  };

  u32x4 qreg[4];
  f32x4 acc[8];
  float m_run, l_part;
  auto reset = [&]() {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegBig;
    l_part = 0.f;
  };
  reset();
  int piece_first = s0;

  auto finish_piece = [&](const RowTile& t, int gidx) {
    float l_row = l_part + __shfl_xor(l_part, 16);
    l_row += __shfl_xor(l_row, 32);
    const int pb = pre[t.b];
    const int nb = pre[t.b + 1] - pb;
    const bool whole = (pb / P) == ((pb + nb - 1) / P);
    if (row_real) {
      const int head = g * G + col;
      if (whole) {
        const float inv = 1.f / l_row;
        uint16_t* op = out + ((int64_t)t.b * HQ + head) * kHeadDim + 4 * grp;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *reinterpret_cast<u32x2*>(op + 16 * db) =
              u32x2{pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv), pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv)};
      } else {
        const int slot = piece_first == s0 ? 0 : 1;
        const int64_t pidx = ((int64_t)blockIdx.x * 2 + slot) * HQ + head;
        float* po = part_o + pidx * kHeadDim + 4 * grp;
#pragma unroll
        for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(po + 16 * db) = acc[db];
        if (grp == 0) {
          part_ml[pidx * 2 + 0] = m_run;
          part_ml[pidx * 2 + 1] = l_row;
        }
      }
    }
    reset();
    piece_first = gidx + 1;
  };

  auto compute = [&](auto stage_c, const RowTile& t, int gi) {
    constexpr int ST = decltype(stage_c)::value;
    const char* kb = rt_lds + ST * kRTStage + g * (kHeadDim * 2);  // head g's 256-byte column of the rows
    const char* vb = kb + kRTTileRows;
    if (t.qload) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qreg[kk] = qst[ST][kk];
    }
    u32x4 kop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kop[kk] = *reinterpret_cast<const u32x4*>(kb + col * kRTRow + 16 * ((4 * kk + grp) ^ col));
    // S^T = K_g Q^T (16 keys x 16 query rows)
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[kk]),
                                                  __builtin_bit_cast(bf16x8, qreg[kk]), s, 0, 0, 0);
    // lane l holds keys 4 grp + i (i = 0..3) of query row col; keys past the context are masked
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = 4 * grp + i < t.nvalid ? s[i] * scale_log2 : -__builtin_inff();
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    const uint32_t w0 = pack_bf16x2(p[0], p[1]);
    const uint32_t w1 = pack_bf16x2(p[2], p[3]);
    // row sum of the weights as rounded to bf16 for the P V products
    l_part = l_part * alpha + ((bf_lo(w0) + bf_hi(w0)) + (bf_lo(w1) + bf_hi(w1)));
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
    // O^T += V_g^T P^T: A = V^T (lane l: dim 16 db + l % 16 of keys 4 grp .. + 3) through the transposing
    // read; lane 4 k + c of a group names key 4 grp + k, dims 16 db + 4 c .. + 3
    const int vk = 4 * grp + ((lane & 15) >> 2);
    const int vc = lane & 3;
    const char* vrow = vb + vk * kRTRow + 8 * (vc & 1);
    const bf16x4 pb4 = __builtin_bit_cast(bf16x4, u32x2{w0, w1});
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint2 va = rt_read_tr16(vrow + 16 * ((2 * db + (vc >> 1)) ^ ((4 * vk) & 15)));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, va), pb4, acc[db], 0, 0, 0);
    }
    // fused store: head g's K and V rows of the sequence's new token go from LDS to its slot
    if constexpr (FUSED) {
      if (nr.k && t.last) {
        const int32_t slot = nr.slots[t.b];
        const int tn = t.nvalid - 1;
        if (slot >= 0 && (int64_t)slot < nr.num_slots && grp == 0) {
          const int64_t dst = (int64_t)slot * kRTRow + g * (kHeadDim * 2);
          *reinterpret_cast<u32x4*>(nr.k_cache + dst + 16 * (col ^ (tn & 15))) =
              *reinterpret_cast<const u32x4*>(kb + tn * kRTRow + 16 * col);
          *reinterpret_cast<u32x4*>(nr.v_cache + dst + 16 * (col ^ ((4 * tn) & 15))) =
              *reinterpret_cast<const u32x4*>(vb + tn * kRTRow + 16 * col);
        }
      }
    }
    if (t.last || gi + 1 == s1) {
      finish_piece(t, gi);
      // vmcnt also counts stores, and loads and stores may complete out of order: wait here for the piece's
      // stores (and the tile in flight), so that the loop's waits can count the loads alone
      __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    }
  };

  // i-th tile of the range in stage ST: issue tile i + 1 into the other stage (which the work-group finished
  // reading at the end of the previous iteration; past the range end the last tile again, so every iteration
  // issues the same eight K/V loads, after any query loads), wait for this wavefront's loads of tile i (vmcnt
  // counts in order: only tile i + 1's eight K/V loads may still be in flight), then a barrier makes the whole
  // tile visible; compute it, and a second barrier frees its stage for tile i + 2
  // (a plain s_barrier: __syncthreads() would also wait for the next tile's loads; the empty asm statements
  // keep the compiler from moving LDS accesses across it)
  auto wg_barrier = []() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };
  RowTile tl[kRTStages];
  auto iteration = [&](auto stage_c, int i) {
    constexpr int ST = decltype(stage_c)::value;
    constexpr int NX = ST ^ 1;
    tl[NX] = i + 1 < n ? next_tile(tl[ST]) : tl[ST];
    issue(RTStage<NX>{}, tl[NX]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(8));
    wg_barrier();
    if (i < n) compute(stage_c, tl[ST], s0 + i);
    wg_barrier();
  };

  tl[0] = make_tile(lo_b, s0 - pre[lo_b]);
  tl[0].qload = 1;
  issue(RTStage<0>{}, tl[0]);
  for (int i = 0; i < n; i += kRTStages) {
    iteration(RTStage<0>{}, i);
    iteration(RTStage<1>{}, i + 1);
  }
}

struct Layout {
  size_t header_bytes, ml_bytes, o_bytes;  // header = steps per wavefront + step prefix
};

// Workspace for `waves` wavefronts (2 partial slots each). The caller-owned
// workspace is sized for the grid cap, so its size does not depend on the
// device; the library's own scratch (paged_attn_decode_noalloc) for the
// launch's actual wavefront count.
Layout workspace_layout(int num_seqs, int num_q_heads, int waves = kWavesCap) {
  Layout lo;
  lo.header_bytes = ((size_t)(num_seqs + 2) * 4 + 255) & ~(size_t)255;
  lo.ml_bytes = ((size_t)waves * 2 * num_q_heads * 2 * 4 + 255) & ~(size_t)255;
  lo.o_bytes = (size_t)waves * 2 * num_q_heads * kHeadDim * 4;
  return lo;
}

// The decode workspace of paged_attn_decode_noalloc: a fixed device array,
// one copy per GPU (allocated when the code object is loaded, held until
// the process ends). 40 MiB covers 32 query heads on 1024 resident
// wavefronts (one work-group of four per CU on 256 CUs).
constexpr size_t kScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

// This device's address of `scratch`, looked up once per device with that
// device current (each GPU holds its own copy at its own address); nullptr
// on error. Host code uses only this address, never the array's name.
char* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return static_cast<char*>(addr[dev]);
}

template <int G, int HKV>
const void* stream_kernel() {  // occupancy is set by the LDS reservation, the same for both forms
  return reinterpret_cast<const void*>(&decode_stream_kernel<G, HKV, false>);
}

const void* pick_kernel(int G, int hkv) {
#define PKV_PICK(GG)                       \
  switch (hkv) {                           \
    case 1: return stream_kernel<GG, 1>(); \
    case 2: return stream_kernel<GG, 2>(); \
    case 4: return stream_kernel<GG, 4>(); \
    default: return stream_kernel<GG, 8>(); \
  }
  switch (G) {  // eight query heads per KV head run on the row-tile kernel or the tile form
    case 1: PKV_PICK(1)
    case 2: PKV_PICK(2)
    default: PKV_PICK(4)
  }
#undef PKV_PICK
}

size_t stream_lds(int num_seqs) {
  const size_t scan = (size_t)(num_seqs + 1) * 4;
  return scan > kStreamLds ? scan : kStreamLds;
}

// Resident work-groups of a decode kernel on the current device (cached per
// device, kernel and LDS size), capped so the partial slots suffice; 0 on error.
int resident_wgs(const void* kernel, size_t lds, int threads = 256) {
  static std::mutex mu;
  static struct Entry {
    int dev;
    const void* k;
    size_t lds;
    int n;
  } cache[128];
  static int ncache = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ncache; ++i)
    if (cache[i].dev == dev && cache[i].k == kernel && cache[i].lds == lds) return cache[i].n;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, lds) != hipSuccess || per < 1) per = 1;
  int n = cus * per;
  if (n * 4 > kWavesCap) n = kWavesCap / 4;  // partial slots are sized for kWavesCap wavefronts (or work-groups)
  if (ncache < 128) cache[ncache++] = Entry{dev, kernel, lds, n};
  return n;
}


template <int G, bool FUSED>
const void* rowtile_kernel() {
  return reinterpret_cast<const void*>(&decode_rowtile_kernel<G, FUSED>);
}

size_t rowtile_lds(int G, int num_seqs) { return (size_t)rt_lds_fixed(G) + (size_t)(num_seqs + 1) * 4; }

// Resident work-groups of the row-tile kernel (one per CU: its two LDS stages take 128 KiB).
int rowtile_grid(int G, int num_seqs) { return resident_wgs(rowtile_kernel<8, false>(), rowtile_lds(G, num_seqs), 512); }

// Whether the row-tile kernel takes a call with these heads and sequences (eight query heads per KV head,
// eight KV heads; its LDS scan holds up to kRTMaxSeqs sequences).
bool rowtile_fits(int G, int num_kv_heads, int num_seqs) {
  return num_kv_heads == kRTKv && G == 8 && num_seqs <= kRTMaxSeqs;
}

// The row-tile decode (decode_rowtile_kernel) and the merge of its partials. `wsb` is the workspace laid out
// as `lo` for `grid` work-groups (two partial slots each).
pkv_status rowtile_call(uint16_t* o, const uint16_t* qq, const char* kc, const char* vc, const int32_t* block_tables,
                        int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs, int G,
                        int64_t num_blocks, float scale_log2, int32_t max_context_len, int grid, char* wsb,
                        const Layout& lo, hipStream_t s, const NewRows& nr);

}  // namespace

bool decode_prepare(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs) {
  if (num_kv_heads < 1 || num_q_heads < num_kv_heads || num_q_heads % num_kv_heads || num_seqs < 1) return false;
  const int G = num_q_heads / num_kv_heads;
  if (rowtile_fits(G, num_kv_heads, num_seqs) && rowtile_grid(G, num_seqs) <= 0) return false;
  if (G == 8) return true;  // the tile form queries nothing
  return resident_wgs(pick_kernel(G, num_kv_heads), stream_lds(num_seqs)) > 0;
}

}  // namespace pkv

extern "C" size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t max_context_len) {
  using namespace pkv;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != kHeadDim || max_context_len < 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  const Layout lo = workspace_layout(num_seqs, num_q_heads);
  return lo.header_bytes + lo.ml_bytes + lo.o_bytes;
}

namespace pkv {
namespace {

// use_scratch: the workspace is the library's `scratch` array
// (paged_attn_decode_noalloc; workspace and workspace_bytes are ignored).
pkv_status decode_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, float scale, int32_t max_context_len, void* workspace,
                       size_t workspace_bytes, void* stream, const NewRows& nr, bool use_scratch = false) {
  if (num_seqs < 0 || num_blocks < 0 || max_context_len < 0 || block_table_stride < 0)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: negative size");
  if (head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: head_dim %d (128 only)", head_dim);
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: block_size %d (256 only)", block_size);
  if (num_kv_heads != 1 && num_kv_heads != 2 && num_kv_heads != 4 && num_kv_heads != 8)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: num_kv_heads %d (1, 2, 4 or 8)", num_kv_heads);
  if (num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: head counts %d/%d unsupported", num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: %d query heads per KV head (1, 2, 4 or 8)", G);
  if (!(scale > 0.f) || !__builtin_isfinite(scale))
    return fail(PKV_ERR_INVALID, "paged_attn_decode: scale must be finite and > 0");
  if (num_seqs == 0) return ok();
  if (num_seqs > kMaxSeqs) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: more than %d sequences", kMaxSeqs);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: q, out and caches must be 16-byte aligned");
  const int64_t need_bt = (max_context_len + kBlockSize - 1) / kBlockSize;
  if (block_table_stride < need_bt)
    return fail(PKV_ERR_INVALID, "paged_attn_decode: block_table_stride %d < %lld blocks of max_context_len",
                block_table_stride, (long long)need_bt);
  // the kernels count two-token steps (a step holds at least two tokens) in 32-bit integers
  if ((int64_t)num_seqs * ((max_context_len + 1) / 2) > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: num_seqs x max_context_len / 2 exceeds 2^31 - 1 steps");
  if (!use_scratch) {
    const size_t ws =
        paged_attn_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len);
    if (!workspace || workspace_bytes < ws)
      return fail(PKV_ERR_WORKSPACE, "paged_attn_decode: workspace of %zu bytes needed, got %zu", ws,
                  workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255)
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: workspace must be 256-byte aligned");
  }

  // The MFMA forms take eight query heads per KV head (the tile form, decode_tile_call, or the row-tile
  // kernel), where the row-wide kernel below is bound by its vector arithmetic (4.0-4.3 TB/s), and the tile
  // form takes small calls with two or four, where the row-wide kernel's fixed cost (two launches, a merge over
  // pieces spread across all wavefronts) dominates.
  // Measured on MI355X, 64 Q / 8 KV, row-wide -> tile form: 1 sequence of 100-2048 tokens 22.0 -> 13.1 us,
  // 16: 45.8 -> 20.7, 256: 282.5 -> 223.5 us; 4096-32768 tokens, 1 sequence 56.1 -> 45.8 us, 128: 2197 -> 1754
  // us. 16 Q / 8 KV, a 28-layer decode step with the store fused, each layer its own caches: contexts of
  // 100-1024 tokens, 16-48 sequences 5-10 % faster on the tile form, 64 sequences 6 % slower; contexts of
  // 1024-2048 tokens, 8-64 sequences 5-17 % slower; 1-4 sequences of any length level or faster. 32 Q / 8 KV,
  // the same step: 100-1024 tokens, 48-80 sequences 1-17 % faster on the tile form, 96 and 128 9-14 % slower;
  // 100-2048 tokens, 8-32 sequences 1-12 % faster, 48 and 64 4-13 % slower; 100-4096 tokens, 8-32 sequences
  // 5-13 % slower.
  // With eight query heads per KV head and eight KV heads, calls that stream longer contexts over enough
  // sequences, or shorter contexts (beyond 768 or 512 tokens) over more sequences, take the row-tile kernel (decode_rowtile_kernel): a 28-layer decode step with the store fused,
  // each layer its own caches, 64 Q / 8 KV, tile form -> row-tile kernel: contexts of 100-2048 tokens, 40-48
  // sequences 1-2 % faster, 64-256 6-12 % faster, 32 or fewer 6-28 % slower; 100-4096 tokens, 48 sequences 15 %
  // faster, 16-32 3-9 % slower; 1024-8192 tokens, 8-64 sequences 8-20 % faster; 100-1024 tokens, 48 sequences
  // 5 % slower, 64-112 3-7 % faster; 512-1024 tokens, 48-64 sequences 3 % slower, 80-112 2-9 % faster; 256-1024
  // and 700-1024 tokens, 80 sequences 7-9 % faster; 100-900 tokens, 80 sequences 3 % slower, 96 3 % faster; at 128
  // sequences and more, contexts of 100-640, 100-768, 100-1024, 256-768, 400-640 and 512-1024 tokens 2-10 % faster
  // (up to 1024 sequences; 256 of 100-640 tokens 2 % slower), 100-512 tokens 128-256 sequences 4 % faster to 6 %
  // slower.
  // PKV_DECODE_FORM=tile, =rowwide or =rowtile in the environment overrides the choice (read on every call;
  // for tests and tuning; eight query heads per KV head never take the row-wide kernel, and the row-tile
  // kernel needs eight KV heads)
  const char* form = getenv("PKV_DECODE_FORM");
  const bool force_tile = form && !strcmp(form, "tile");
  const bool force_rowwide = form && !strcmp(form, "rowwide");
  const bool force_rowtile = form && !strcmp(form, "rowtile");
  const bool small_call =
      num_seqs <= kTileFewSeqs ||
      (num_seqs <= (G == 4 ? kTileShortSeqsG4 : kTileShortSeqs) && max_context_len <= kTileShortCtx) ||
      (G == 4 && num_seqs <= kTileMidSeqsG4 && max_context_len <= kTileMidCtx);
  // the row-tile kernel counts 16-token tiles in 32-bit integers
  const bool rowtile_ok = rowtile_fits(G, num_kv_heads, num_seqs) &&
                          (int64_t)num_seqs * ((max_context_len + kRT - 1) / kRT) <= INT32_MAX;
  const bool rowtile_pick = G == 8 && ((num_seqs >= kRowTileSeqs && max_context_len > kRowTileCtx) ||
                                       (num_seqs >= kRowTileLongSeqs && max_context_len > kRowTileLongCtx) ||
                                       (num_seqs >= kRowTileMidSeqs && max_context_len > kRowTileMidCtx) ||
                                       (num_seqs >= kRowTileManySeqs && max_context_len > kRowTileManyCtx));
  if (rowtile_ok && (force_rowtile || (rowtile_pick && !force_tile))) {
    const int grid = rowtile_grid(G, num_seqs);
    if (grid <= 0) return fail(PKV_ERR_HIP, "paged_attn_decode: cannot query the device");
    Layout lo;
    char* wsb;
    if (use_scratch) {
      lo = workspace_layout(num_seqs, num_q_heads, grid);
      const size_t need = lo.header_bytes + lo.ml_bytes + lo.o_bytes;
      if (need > kScratchBytes)
        return fail(PKV_ERR_UNSUPPORTED,
                    "paged_attn_decode_noalloc: %d query heads on %d work-groups need %zu bytes of workspace, more "
                    "than the library's %zu-byte scratch", num_q_heads, grid, need, kScratchBytes);
      wsb = scratch_address();
      if (!wsb) return fail(PKV_ERR_HIP, "paged_attn_decode_noalloc: cannot find the device's scratch array");
    } else {
      lo = workspace_layout(num_seqs, num_q_heads);
      wsb = static_cast<char*>(workspace);
    }
    return rowtile_call(static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
                        static_cast<const char*>(k_cache), static_cast<const char*>(v_cache), block_tables,
                        block_table_stride, context_lens, num_seqs, G, num_blocks, scale * 1.4426950408889634f,
                        max_context_len, grid, wsb, lo, reinterpret_cast<hipStream_t>(stream), nr);
  }
  if (G == 8 || (G >= 2 && !force_rowwide && (force_tile || small_call))) {
    void* tws = workspace;
    size_t tws_bytes = workspace_bytes;
    if (use_scratch) {
      tws = scratch_address();
      tws_bytes = kScratchBytes;
      if (!tws) return fail(PKV_ERR_HIP, "paged_attn_decode_noalloc: cannot find the device's scratch array");
    }
    return decode_tile_call(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs,
                            num_q_heads, num_kv_heads, num_blocks, scale, max_context_len, tws, tws_bytes, stream,
                            nr);
  }

  const float scale_log2 = scale * 1.4426950408889634f;
  const size_t lds = stream_lds(num_seqs);
  // Part of the CUs, by the query heads per KV head: measured on MI355X (256 CUs) with 192, 224 and 256
  // work-groups, one or two query heads per KV head (a step's arithmetic is light) ran fastest on 192 at
  // every context length tried (U[100, 2048] to U[4096, 32768]; 2-6 % ahead of 256), four (twice the
  // arithmetic per byte) on all 256 (5-15 % ahead of 192).
  const int resident = resident_wgs(pick_kernel(G, num_kv_heads), lds);
  if (resident <= 0) return fail(PKV_ERR_HIP, "paged_attn_decode: cannot query the device");
  const int grid = resident < 8 || G >= 4 ? resident : resident * 3 / 4;

  Layout lo;
  char* wsb;
  if (use_scratch) {
    lo = workspace_layout(num_seqs, num_q_heads, grid * 4);
    const size_t need = lo.header_bytes + lo.ml_bytes + lo.o_bytes;
    if (need > kScratchBytes)
      return fail(PKV_ERR_UNSUPPORTED,
                  "paged_attn_decode_noalloc: %d query heads on %d wavefronts need %zu bytes of workspace, more "
                  "than the library's %zu-byte scratch (use paged_attn_decode with a caller workspace)",
                  num_q_heads, grid * 4, need, kScratchBytes);
    wsb = scratch_address();
    if (!wsb) return fail(PKV_ERR_HIP, "paged_attn_decode_noalloc: cannot find the device's scratch array");
  } else {
    lo = workspace_layout(num_seqs, num_q_heads);
    wsb = static_cast<char*>(workspace);
  }
  int32_t* header = reinterpret_cast<int32_t*>(wsb);
  float* part_ml = reinterpret_cast<float*>(wsb + lo.header_bytes);
  float* part_o = reinterpret_cast<float*>(wsb + lo.header_bytes + lo.ml_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* o = static_cast<uint16_t*>(out);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
#define PKV_DECODE_LAUNCH(GG, HH, LZ)                                                                     \
  hipLaunchKernelGGL((decode_stream_kernel<GG, HH, LZ>), dim3(grid), dim3(256), lds, s, o, qq, kc, vc,   \
                     block_tables, block_table_stride, context_lens, num_seqs, num_blocks, scale_log2,   \
                     max_context_len, header, part_ml, part_o, nr)
#define PKV_DECODE_HKV(GG, LZ)                    \
  switch (num_kv_heads) {                         \
    case 1: PKV_DECODE_LAUNCH(GG, 1, LZ); break;  \
    case 2: PKV_DECODE_LAUNCH(GG, 2, LZ); break;  \
    case 4: PKV_DECODE_LAUNCH(GG, 4, LZ); break;  \
    default: PKV_DECODE_LAUNCH(GG, 8, LZ); break; \
  }
  // lazy rescale: four query heads per KV head over long contexts (measured: 2.6 % faster on 512 sequences
  // of 4096-32768 tokens, 3.7 % slower on contexts up to 2048)
  switch (G) {
    case 1: PKV_DECODE_HKV(1, false) break;
    case 2: PKV_DECODE_HKV(2, false) break;
    case 4:
      if (max_context_len > 4096) {
        PKV_DECODE_HKV(4, true)
      } else {
        PKV_DECODE_HKV(4, false)
      }
      break;
    default: return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: %d query heads per KV head", G);
  }
#undef PKV_DECODE_HKV
#undef PKV_DECODE_LAUNCH
  pkv_status st = check_launch("paged_attn_decode (stream)");
  if (st != PKV_OK) return st;
  switch (num_q_heads) {  // HQ = G * H_kv, both powers of two up to 8
#define PKV_MERGE(HQV)                                                                                  \
  case HQV:                                                                                             \
    if (num_seqs <= kWideMergeMaxSeqs)                                                                  \
      hipLaunchKernelGGL((decode_merge_wide_kernel<HQV>), dim3(num_seqs, HQV), dim3(1024), 0, s, o, header, \
                         part_ml, part_o, context_lens);                                               \
    else                                                                                                \
      hipLaunchKernelGGL((decode_merge_kernel<HQV>), dim3(num_seqs), dim3(HQV * 16), 0, s, o, header,     \
                         part_ml, part_o, context_lens);                                                \
    break;
    PKV_MERGE(1) PKV_MERGE(2) PKV_MERGE(4) PKV_MERGE(8) PKV_MERGE(16) PKV_MERGE(32) PKV_MERGE(64)
#undef PKV_MERGE
    default: return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: %d query heads", num_q_heads);
  }
  return check_launch("paged_attn_decode (merge)");
}

pkv_status rowtile_call(uint16_t* o, const uint16_t* qq, const char* kc, const char* vc, const int32_t* block_tables,
                        int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs, int G,
                        int64_t num_blocks, float scale_log2, int32_t max_context_len, int grid, char* wsb,
                        const Layout& lo, hipStream_t s, const NewRows& nr) {
  int32_t* header = reinterpret_cast<int32_t*>(wsb);
  float* part_ml = reinterpret_cast<float*>(wsb + lo.header_bytes);
  float* part_o = reinterpret_cast<float*>(wsb + lo.header_bytes + lo.ml_bytes);
  const size_t lds = rowtile_lds(G, num_seqs);
#define PKV_RT_LAUNCH(GG, FF)                                                                                  \
  hipLaunchKernelGGL((decode_rowtile_kernel<GG, FF>), dim3(grid), dim3(512), lds, s, o, qq, kc, vc, block_tables, \
                     block_table_stride, context_lens, num_seqs, num_blocks, scale_log2, max_context_len, header, \
                     part_ml, part_o, nr)
  if (nr.k)
    PKV_RT_LAUNCH(8, true);
  else
    PKV_RT_LAUNCH(8, false);
#undef PKV_RT_LAUNCH
  pkv_status st = check_launch("paged_attn_decode (row tiles)");
  if (st != PKV_OK) return st;
  // 64 query heads (G = 8 on eight KV heads)
  if (num_seqs <= kWideMergeMaxSeqs)
    hipLaunchKernelGGL((decode_merge_wide_kernel<64>), dim3(num_seqs, 64), dim3(1024), 0, s, o, header, part_ml,
                       part_o, context_lens);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(num_seqs), dim3(64 * 16), 0, s, o, header, part_ml, part_o,
                       context_lens);
  return check_launch("paged_attn_decode (row-tile merge)");
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t block_table_stride,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int64_t num_blocks, float scale, int32_t max_context_len, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  const pkv::NewRows none{nullptr, nullptr, 0, 0, nullptr, 0, nullptr, nullptr};
  return pkv::decode_call(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, max_context_len,
                          workspace, workspace_bytes, stream, none);
}

extern "C" pkv_status paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                                const int32_t* block_tables, int32_t block_table_stride,
                                                const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                int64_t num_blocks, float scale, int32_t max_context_len,
                                                void* stream) {
  const pkv::NewRows none{nullptr, nullptr, 0, 0, nullptr, 0, nullptr, nullptr};
  return pkv::decode_call(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, max_context_len,
                          nullptr, 0, stream, none, true);
}

extern "C" pkv_status paged_attn_decode_store(void* out, const void* q, const void* key, int64_t key_token_stride,
                                              const void* value, int64_t value_token_stride,
                                              const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                              const int32_t* block_tables, int32_t block_table_stride,
                                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int64_t num_blocks, float scale, int32_t max_context_len,
                                              void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (num_seqs > 0) {
    if (!key || !value || !slot_mapping) return fail(PKV_ERR_INVALID, "paged_attn_decode_store: null pointer");
    if (head_dim != kHeadDim)
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode_store: head_dim %d (128 only)", head_dim);
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (key_token_stride < row || value_token_stride < row)
      return fail(PKV_ERR_INVALID, "paged_attn_decode_store: token stride smaller than a row (%lld elements)",
                  (long long)row);
    if ((key_token_stride * 2) % 16 || (value_token_stride * 2) % 16 || !aligned16(key) || !aligned16(value))
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode_store: key/value and their strides must be 16-byte aligned");
    if (num_blocks > INT64_MAX / block_size || block_size <= 0)
      return fail(PKV_ERR_INVALID, "paged_attn_decode_store: num_blocks or block_size out of range");
  }
  const NewRows nr{static_cast<const char*>(key), static_cast<const char*>(value), key_token_stride * 2,
                   value_token_stride * 2, slot_mapping, num_blocks * (block_size > 0 ? block_size : 1),
                   static_cast<char*>(k_cache), static_cast<char*>(v_cache)};
  return decode_call(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, max_context_len, workspace,
                     workspace_bytes, stream, nr);
}
