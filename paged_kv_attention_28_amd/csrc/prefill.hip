// paged_attn_prefill_varlen: causal varlen attention whose queries start at
// num_cached_tokens, keys read through the block table.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm": the step computes only tokens from
// num_cached onward ("第二站：一个请求的状态"); with a prefix hit or a chunk
// continuation the whole context is read from the paged cache through the
// block table ("第六站：注意力层"); only the first sequence of a step may be a
// chunk cut at an arbitrary point ("第三站：调度器").
//
// gfx950 design (the two genuinely dense contractions run on MFMA):
//  * Work-group = 4 wavefronts on 128 (token, head) rows of one sequence and
//    one KV head: 128 / G query tokens x the G query heads sharing that KV
//    head, so each K/V tile staged in LDS serves every one of them.
//  * Work items come from a host plan (pkv_prefill_plan): one per non-empty
//    (sequence, q-tile, kv_head), longest first, KV heads of a tile adjacent,
//    so no work-group is launched for nothing, the short tiles fill the tail,
//    and (with round-robin dispatch over the 8 XCDs) all tiles of one KV head
//    land on one XCD and share its L2. Without a plan the grid is (kv_head,
//    seq, q-tile counted from the end), sized by max_q_len, and work-groups
//    past a sequence's last tile exit at once.
//  * Per 32-key tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows
//    from LDS, B = the wavefront's 32 query rows held in registers). In the
//    transposed product each lane holds 16 scores of one query row, so the
//    row max and sum need a single cross-lane exchange (lane ^ 32).
//  * Occupancy: with 32-key tiles the kernel needs 164 VGPRs and 32 KiB of
//    LDS, so three work-groups (three wavefronts per SIMD) share a CU; the
//    third wavefront hides the latencies of the LDS operand reads, the MFMA
//    chains and the per-tile barrier. (The loops also take 64-key tiles,
//    kSub = 2, at two work-groups per CU: 10 % slower.)
//  * O^T += V^T P^T, again 32x32x16: B = P taken straight from the S^T
//    accumulators (rounded to bf16) because the K rows were fed to the first
//    product in a permuted order (bits 2 and 3 of the row index swapped)
//    that makes each lane's 8 scores belong to 8 consecutive keys; A = V^T,
//    read from the row-major V tile with gfx950's transposing LDS load
//    (ds_read_b64_tr_b16), so V is staged exactly like K.
//  * fp32 online softmax in the log2 domain with lazy rescaling (the
//    reference max moves only when a row max exceeds it by 8, so most tiles
//    skip rescaling the 64 output accumulators); the row sum adds the
//    weights as rounded to bf16 for the P V products; a wavefront skips the
//    tiles above its last query row.
//  * K/V of tile i+1 go from the cache straight into LDS (buffer loads with
//    the lds bit, buffer_load_dwordx4 ... lds: a scalar descriptor per tile
//    and loop-invariant 32-bit lane offsets) while tile i is computed: no
//    registers, no LDS writes by the wavefronts; two LDS buffers, one wait
//    and one barrier per tile. Such a load writes lane l's 16 bytes at LDS
//    base + 16 l, so
//    rows cannot be padded; instead the 16-byte chunks of each 256-byte row
//    are XOR-swizzled (by r % 16 in K, by 4 r % 16 in V), which keeps the
//    16-byte K reads and the transposing V reads free of bank conflicts.
//  * Keys past the context end are clamped to the last context row (a valid,
//    written row) and masked, so stale cache rows never enter the result.
//  * Few vector instructions besides the math: the key loop is unrolled over
//    its two LDS stages, so each stage's base is an immediate offset of the
//    operand reads and the tile loads take scalar LDS destinations; the
//    lane ^ 32 row-max exchange is one v_permlane32_swap (no LDS round trip);
//    block ids are bounds-checked with one unsigned 32-bit scalar compare.
//  * K operands are read four ahead of the S^T products (schedule pinned with
//    sched_group_barrier), and the P V^T products run key-chunk outer, so the
//    second half of the exponentials overlaps the first four products.
//  * A decode form (decode_tile_call) runs the same kernel with each
//    sequence's one new token as the query, one work-group per (KV head,
//    sequence): decode with eight query heads per KV head, whose arithmetic
//    per byte is too heavy for the row-wide decode kernel's vector FMAs.
//  * The output leaves through LDS: the accumulators hold O^T (a lane owns one
//    query row, 8-byte runs of dims), so each wavefront stages its 32 rows in
//    LDS and writes whole 256-byte rows, 16 bytes per lane; stored directly,
//    every store instruction would touch 32 rows 16 bytes at a time. The row
//    stores are nontemporal (streaming).

#include "common.h"

namespace pkv {

namespace {

constexpr int kKeysPerTile = 32;
constexpr int kSub = kKeysPerTile / 32;     // 32-key subtiles per tile
constexpr int kRowsW = kKeysPerTile / 4;    // tile rows each wavefront loads
constexpr int kRowBytes = kHeadDim * 2;               // one head of one key: 256 B
constexpr int kTileBytes = kKeysPerTile * kRowBytes;   // a K (or V) tile: 8 KiB, rows unpadded
constexpr float kNegBig = -1e30f;
constexpr int kPartStride = 4 + kHeadDim;  // floats per (head, chunk) partial of the split decode form
constexpr int64_t kTileDecodeTargetWgs = 1536;  // the split decode form's work-group target (2 x 3 per CU x 256)
constexpr float kRescaleSlack = 8.f;  // log2 units: the reference max moves only when a row max exceeds it by this

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int perm_row(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4k + c names row k, 4-element chunk c; lane i receives element i of the
// group's 4 x 16 block from rows 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* __restrict__ p) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
#pragma clang diagnostic pop
  return __builtin_bit_cast(uint2, v);
}

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
struct Stage {
  static constexpr int value = N;
};

// c + the two bf16 halves of w (v_dot2_f32_bf16 against 1.0, 1.0)
__device__ __forceinline__ float dot2_ones(uint32_t w, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), c,
                                         false);
}

// max of x over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip)
__device__ __forceinline__ float max_lane32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// K and V of keys [key0, key0 + kKeysPerTile) straight from the cache into
// LDS (buffer_load_dwordx4 with the lds bit: lane l of an instruction writes
// its 16 bytes at LDS base + 16 l, whatever address it loads; the descriptor
// bounds the reads to the tile). Wavefront w moves rows kRowsW w ..
// kRowsW (w + 1) - 1, four rows per instruction. Rows are stored unpadded,
// with their 16-byte chunks XOR-swizzled so that the operand reads hit
// distinct banks: physical chunk p of row r holds logical chunk p ^ (r % 16)
// in K and p ^ (4 r % 16) in V. Keys past the context end load its last row.
__device__ __forceinline__ void issue_tile(char* kbuf, char* vbuf, const char* __restrict__ kc,
                                           const char* __restrict__ vc, int32_t blk32, int key0, int L,
                                           int64_t row_bytes, int64_t block_bytes, int head_off,
                                           uint32_t num_blocks32, int wave, const uint32_t (&koff)[4],
                                           const uint32_t (&voff)[4]) {
  // caller error: stay inside the pool (one unsigned compare also rejects negative ids)
  const int64_t blk = (uint32_t)blk32 < num_blocks32 ? (int64_t)(uint32_t)blk32 : 0;
  // wave-uniform start of the tile in both caches; lanes add 32-bit offsets
  const int64_t base = blk * block_bytes + (int64_t)(key0 & (kBlockSize - 1)) * row_bytes + head_off;
  const int span = kKeysPerTile * (int)row_bytes;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0, span, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0, span, 0x00020000);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  if (key0 + kKeysPerTile <= L) {
#pragma unroll
    for (int i = 0; i < kRowsW / 4; ++i) {
      const int r0 = kRowsW * wave + 4 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kbuf + r0 * kRowBytes), 16, koff[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vbuf + r0 * kRowBytes), 16, voff[i], 0, 0, 0);
    }
  } else {
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 4;
    const int last = L - 1 - key0;  // >= 0: the tile starts inside the context
#pragma unroll
    for (int i = 0; i < kRowsW / 4; ++i) {
      const int r0 = kRowsW * wave + 4 * i;
      const int r = r0 + sub;
      const int back = r > last ? r - last : 0;  // rows to step back to the last context row
      const uint32_t d = (uint32_t)back * (uint32_t)row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kbuf + r0 * kRowBytes), 16, koff[i] - d, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vbuf + r0 * kRowBytes), 16, voff[i] - d, 0, 0, 0);
    }
  }
#pragma clang diagnostic pop
}

// The step's new K/V rows (NewRows, common.h) for the fused store
// (paged_attn_prefill_store): positions >= num_cached of a sequence are read
// from the step's key/value input (token q0 + p - c of the step) instead of
// the cache, and each work-group writes its own query tokens' rows of its KV
// head to their slots.

// issue_tile for a tile that holds new tokens: rows r < cut (positions < c)
// from the cache (descriptor as in issue_tile), rows r >= cut from the
// step's input rows, whose tile row r is at kin / vin + (r - rs) * stride
// (rs = max(cut, 0), the first input row); input rows past the context end
// load its last row. Chunks are swizzled as in issue_tile. A row's source is
// chosen per 16-lane group with the exec mask, so each load writes only its
// rows' LDS locations.
__device__ __forceinline__ void issue_tile_new(char* kbuf, char* vbuf, const char* __restrict__ kc,
                                               const char* __restrict__ vc, int32_t blk32, int key0, int L, int cut,
                                               int64_t row_bytes, int64_t block_bytes, int head_off,
                                               uint32_t num_blocks32, int wave, const uint32_t (&koff)[4],
                                               const uint32_t (&voff)[4], const char* kin, const char* vin,
                                               uint32_t ks, uint32_t vs) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;
  const int cp = lane & 15;
  const int last = L - 1 - key0;  // >= cut: the context's last position is a new token
  const int rs = cut > 0 ? cut : 0;
  const __amdgpu_buffer_rsrc_t ki = __builtin_amdgcn_make_buffer_rsrc((void*)kin, (short)0, kKeysPerTile * ks, 0x00020000);
  const __amdgpu_buffer_rsrc_t vi = __builtin_amdgcn_make_buffer_rsrc((void*)vin, (short)0, kKeysPerTile * vs, 0x00020000);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
  if (cut > 0) {  // straddles the cached prefix: its first rows come from the cache
    const int64_t blk = (uint32_t)blk32 < num_blocks32 ? (int64_t)(uint32_t)blk32 : 0;
    const int64_t base = blk * block_bytes + (int64_t)(key0 & (kBlockSize - 1)) * row_bytes + head_off;
    const int span = kKeysPerTile * (int)row_bytes;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0, span, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0, span, 0x00020000);
#pragma unroll
    for (int i = 0; i < kRowsW / 4; ++i) {
      const int r0 = kRowsW * wave + 4 * i;
      if (r0 + sub < cut) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kbuf + r0 * kRowBytes), 16, koff[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vbuf + r0 * kRowBytes), 16, voff[i], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsW / 4; ++i) {
    const int r0 = kRowsW * wave + 4 * i;
    const int r = r0 + sub;
    if (r >= cut) {
      // input row of tile row r (rows past the context end: its last row), relative to the first input row
      const uint32_t ri = (uint32_t)((r < last ? r : last) - rs);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ki, (lds_void*)(kbuf + r0 * kRowBytes), 16,
                                               ri * ks + 16 * (cp ^ (r & 15)), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vi, (lds_void*)(vbuf + r0 * kRowBytes), 16,
                                               ri * vs + 16 * (cp ^ ((4 * r) & 15)), 0, 0, 0);
    }
  }
#pragma clang diagnostic pop
}

// DECODE: the decode form (decode_tile_call). The grid is (KV head,
// sequence); the query is the sequence's one new token (row s of q and out,
// position context_lens[s] - 1), so only the first wavefront holds query
// rows (the others still move their share of every tile); an empty context
// gives zero output rows.
template <int G, bool FUSED, bool DECODE = false>
__global__ __launch_bounds__(256, kKeysPerTile == 32 ? 3 : 2) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_seqlens_q,
    const int32_t* __restrict__ context_lens, const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, int bt_stride, int hq, int hkv, int64_t num_blocks,
    float scale_log2, int max_q, int max_ctx, const int2* __restrict__ items, int num_seqs, const NewRows nr,
    int chunk_tiles = 0, float* __restrict__ part = nullptr) {
  constexpr int kTokWG = 128 / G;  // query tokens per work-group
  constexpr int kTokW = 32 / G;    // per wavefront
  // K0 V0 K1 V1; after the last tile, the output staging (32 rows per wavefront)
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes > 4 * 32 * kRowBytes ? 4 * kTileBytes
                                                                                       : 4 * 32 * kRowBytes];
  __shared__ int32_t own_slots[FUSED ? kTokWG : 1];  // fused store: the slots of this work-group's query tokens

  // work item: the decode form's (kv_head, seq) grid; else from the host plan
  // (one per non-empty tile, heaviest first), else from the grid (kv_head,
  // seq, q-tile counted from the end)
  int g, b, tile;
  if (DECODE) {
    g = blockIdx.x;
    b = blockIdx.y;
    tile = 0;
  } else if (items) {
    const int2 it = items[blockIdx.x];
    b = it.x;
    g = it.y & 255;
    tile = it.y >> 8;
    if (b < 0 || b >= num_seqs || g >= hkv || tile < 0) return;
  } else {
    g = blockIdx.x;
    b = blockIdx.y;
    tile = -1 - (int)blockIdx.z;  // resolved once the tile count is known
  }
  const int q0 = DECODE ? b : cu_seqlens_q[b];
  int n = DECODE ? 1 : cu_seqlens_q[b + 1] - q0;
  n = n > max_q ? max_q : n;
  int L = context_lens[b];
  L = L > max_ctx ? max_ctx : L;
  if (DECODE && L <= 0) {  // empty context: zero output for this KV head's query heads
    if ((int)threadIdx.x < 16 * G) {
      const int h = (int)threadIdx.x >> 4;
      *reinterpret_cast<u32x4*>(out + ((int64_t)b * hq + g * G + h) * kHeadDim + 8 * (threadIdx.x & 15)) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const int c = L - n;
  if (n <= 0 || c < 0) return;
  const int ntiles = (n + kTokWG - 1) / kTokWG;
  if (tile < 0) tile += ntiles;
  if (tile < 0 || tile >= ntiles) return;
  const int tok_begin = tile * kTokWG;
  const int tok_end = tok_begin + kTokWG < n ? tok_begin + kTokWG : n;
  const int kv_end = c + tok_end;
  int nkt = (kv_end + kKeysPerTile - 1) / kKeysPerTile;
  // decode form split over the keys (chunk_tiles > 0): this work-group takes key tiles [kt0, nkt) of chunk
  // blockIdx.z and leaves unnormalised partials; chunks past the context have nothing to do
  int kt0 = 0;
  if (DECODE && chunk_tiles > 0) {
    kt0 = (int)blockIdx.z * chunk_tiles;
    if (kt0 >= nkt) return;
    nkt = kt0 + chunk_tiles < nkt ? kt0 + chunk_tiles : nkt;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;  // query row of this lane in the wavefront's 32 rows
  const int half = lane >> 5;

  // wavefront's rows and query positions
  const int wtok0 = tok_begin + wave * kTokW;
  const bool wave_live = wtok0 < tok_end;
  const int wtok1 = wtok0 + kTokW < tok_end ? wtok0 + kTokW : tok_end;
  const int pmin = c + wtok0;
  const int pmax = c + wtok1 - 1;

  const int r = wave * 32 + col;
  const int tok = tok_begin + r / G;
  const bool row_valid = tok < tok_end;
  const int tokc = row_valid ? tok : tok_end - 1;
  const int qhead = g * G + (r % G);
  const int pos = c + tokc;

  // query rows as the B operand of S^T = K Q^T: dims 16 kk + 8 half .. +7
  u32x4 qreg[8];
  {
    const uint16_t* qp = q + ((int64_t)(q0 + tokc) * hq + qhead) * kHeadDim + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = *reinterpret_cast<const u32x4*>(qp + 16 * kk);
  }

  f32x16 acc_o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_o[dt][i] = 0.f;
  float m_ref = kNegBig;  // reference max (log2 domain) of this lane's row
  float l_run = 0.f;

  const int64_t row_bytes = (int64_t)hkv * kHeadDim * 2;
  const int64_t block_bytes = row_bytes * kBlockSize;
  const int head_off = g * kRowBytes;
  const int32_t* bt = block_tables + (int64_t)b * bt_stride;
  // loop-invariant lane offsets (bytes from the tile start) of the rows this lane loads
  uint32_t gk[4], gv[4];
  {
    const int sub = lane >> 4;
    const int cp = lane & 15;
#pragma unroll
    for (int i = 0; i < kRowsW / 4; ++i) {
      const int r = kRowsW * wave + 4 * i + sub;
      gk[i] = (uint32_t)r * (uint32_t)row_bytes + 16 * (cp ^ (r & 15));
      gv[i] = (uint32_t)r * (uint32_t)row_bytes + 16 * (cp ^ ((4 * r) & 15));
    }
  }
  const uint32_t nblk32 = num_blocks > 0x7fffffff ? 0x7fffffffu : (uint32_t)num_blocks;
  // fused store: the input row of position c (token q0 of the step), this KV head
  const char* kin0 = nullptr;
  const char* vin0 = nullptr;
  uint32_t ks = 0, vs = 0;
  if constexpr (FUSED) {
    kin0 = nr.k + (int64_t)q0 * nr.k_stride_b + head_off;
    vin0 = nr.v + (int64_t)q0 * nr.v_stride_b + head_off;
    ks = (uint32_t)nr.k_stride_b;
    vs = (uint32_t)nr.v_stride_b;
  }
  int32_t my_slot = -1;  // fused store: loaded before the first tile is issued, kept in LDS after
  if (FUSED && (int)threadIdx.x < tok_end - tok_begin) my_slot = nr.slots[q0 + tok_begin + threadIdx.x];
  // K/V of the tile starting at key0: from the cache, or (fused store) partly or wholly from the input rows
  auto issue = [&](char* kb, int key0, int32_t blk32) {
    if (!FUSED || key0 + kKeysPerTile <= c) {
      issue_tile(kb, kb + kTileBytes, k_cache, v_cache, blk32, key0, L, row_bytes, block_bytes, head_off, nblk32,
                 wave, gk, gv);
    } else {
      const int cut = c - key0;
      const int64_t first = key0 > c ? key0 - c : 0;  // input row of the tile's first new token
      issue_tile_new(kb, kb + kTileBytes, k_cache, v_cache, blk32, key0, L, cut, row_bytes, block_bytes, head_off,
                     nblk32, wave, gk, gv, kin0 + first * nr.k_stride_b, vin0 + first * nr.v_stride_b, ks, vs);
    }
  };
  issue(smem, kt0 * kKeysPerTile, bt[(kt0 * kKeysPerTile) >> 8]);
  if (FUSED && (int)threadIdx.x < tok_end - tok_begin) own_slots[threadIdx.x] = my_slot;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) retire(qreg[kk]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // per-lane LDS byte offsets of the MFMA operands (swizzle as in issue_tile)
  int koff[8];  // A of S^T: K row perm_row(col), logical chunk 2 kk + half
  {
    const int row = perm_row(col);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) koff[kk] = row * kRowBytes + 16 * ((2 * kk + half) ^ (row & 15));
  }
  int voff[4];  // A of O^T via transposing reads: dims 32 dt .. of rows R0 (+ 32 st + 16 qq + 4 hi)
  {
    const int q16 = lane >> 4;
    const int r0 = 8 * (q16 >> 1) + ((lane & 15) >> 2);
    const int rr = (lane >> 2) & 3;  // r0 % 4: the V swizzle flips chunk bits 2-3 by it
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      voff[dt] = r0 * kRowBytes + 16 * (2 * (q16 & 1) + ((lane & 3) >> 1) + 4 * (dt ^ rr)) + 8 * (lane & 1);
  }

  // one key tile; the LDS stage is a compile-time constant so that operand
  // addresses fold the stage base into the instructions' offset fields
  auto key_tile = [&](auto stage_c, const int kt) {
    constexpr int stg = decltype(stage_c)::value;
    const char* kbuf = smem + stg * 2 * kTileBytes;
    const char* vbuf = kbuf + kTileBytes;
    const int key0 = kt * kKeysPerTile;
    if constexpr (FUSED) {
      // Fused store: this tile's rows of the work-group's own query tokens (positions c + tok_begin ..
      // c + tok_end - 1, read from the input into LDS) go to their slots, head g only; each (token, KV head)
      // belongs to exactly one work-group. Issued before the next tile's loads, so the end-of-tile wait
      // covers these stores too.
      const int own_lo = c + tok_begin - key0 > 0 ? c + tok_begin - key0 : 0;
      const int own_hi = c + tok_end - key0 < kKeysPerTile ? c + tok_end - key0 : kKeysPerTile;
      if (own_lo < own_hi) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));  // keeps the address arithmetic here (hoisted, it would be spilled)
        const int row = tid >> 3;
        const int j = tid & 7;
        if (row >= own_lo && row < own_hi) {
          const int32_t slot = own_slots[key0 + row - c - tok_begin];
          if (slot >= 0 && (int64_t)slot < nr.num_slots) {
            char* kd = nr.k_cache + (int64_t)slot * row_bytes + head_off;
            char* vd = nr.v_cache + (int64_t)slot * row_bytes + head_off;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int ch = 2 * j + h;  // logical 16-byte chunk
              *reinterpret_cast<u32x4*>(kd + 16 * ch) =
                  *reinterpret_cast<const u32x4*>(kbuf + row * kRowBytes + 16 * (ch ^ (row & 15)));
              *reinterpret_cast<u32x4*>(vd + 16 * ch) =
                  *reinterpret_cast<const u32x4*>(vbuf + row * kRowBytes + 16 * (ch ^ ((4 * row) & 15)));
            }
          }
        }
      }
    }
    const bool has_next = kt + 1 < nkt;
    if (has_next) issue(smem + (1 - stg) * 2 * kTileBytes, (kt + 1) * kKeysPerTile, bt[((kt + 1) * kKeysPerTile) >> 8]);
    const bool act0 = wave_live && key0 <= pmax;
    const bool act1 = kSub == 2 && wave_live && key0 + 32 <= pmax;
    if (act0) {
      f32x16 s[kSub];
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        if (st == 1 && !act1) break;
        const char* kr = kbuf + 32 * st * kRowBytes;
        // K operands four reads ahead of the products that use them
        u32x4 a[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const u32x4*>(kr + koff[kk]);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const u32x4 cur = a[kk & 3];
          if (kk + 4 < 8) a[kk & 3] = *reinterpret_cast<const u32x4*>(kr + koff[kk + 4]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(qreg[kk]),
                                                          kk == 0 ? f32x16{} : s[st], 0, 0, 0);
        }
        // keep the schedule: four reads, then product / next read pairs, then the last four products
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      if (kSub == 2 && !act1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kSub - 1][i] = -__builtin_inff();
      }
      // Accumulator element i of subtile st holds key
      //   key0 + 32 st + 16 (i >> 3) + 8 half + (i & 7)
      // (output row 8 (i/4) + 4 half + i%4 of the MFMA, through perm_row).
      if (key0 + kKeysPerTile - 1 > pmin) {  // tile crosses the causal diagonal of some row
        const int lim = pos - key0 - 8 * half;  // element visible iff its key offset <= lim
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * st + 16 * (i >> 3) + (i & 7) > lim) s[st][i] = -__builtin_inff();
      }
      float mx = kNegBig;
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
      mx = max_lane32(mx) * scale_log2;
      // Lazy rescale: exponents are taken against m_ref, which moves (and
      // rescales this row's running sums) only when the row max exceeds it
      // by more than kRescaleSlack, so weights stay <= 2^slack. The decision
      // is per row (other rows keep alpha = 1 exactly), so a row's result
      // never depends on the other rows of the wavefront.
      const bool grow = mx > m_ref + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[dt][i] *= alpha;
        m_ref = m_new;
      }
      u32x4 pk[kSub][2];
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][i], scale_log2, -m_ref));
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          pk[st][qq].x = pack_bf16x2(p[8 * qq + 0], p[8 * qq + 1]);
          pk[st][qq].y = pack_bf16x2(p[8 * qq + 2], p[8 * qq + 3]);
          pk[st][qq].z = pack_bf16x2(p[8 * qq + 4], p[8 * qq + 5]);
          pk[st][qq].w = pack_bf16x2(p[8 * qq + 6], p[8 * qq + 7]);
        }
      }
      // Row sum of the weights as rounded to bf16 for the P V products, so
      // the output is divided by exactly the weights that were applied: with
      // the lazy reference max the largest weight lies anywhere in (1, 256]
      // and its rounding would otherwise show in full in a peaky row's output.
      float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          lsum0 = dot2_ones(pk[st][qq].x, lsum0);
          lsum1 = dot2_ones(pk[st][qq].y, lsum1);
          lsum0 = dot2_ones(pk[st][qq].z, lsum0);
          lsum1 = dot2_ones(pk[st][qq].w, lsum1);
        }
      l_run += lsum0 + lsum1;
      // key chunk outer, output dims inner: the four products of the first 16
      // keys need only the first half of the weights, so the second half's
      // exponentials can run while they execute
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        if (st == 1 && !act1) break;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const char* vr = vbuf + (32 * st + 16 * qq) * kRowBytes + voff[dt];
            const uint2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vr));
            const uint2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vr + 4 * kRowBytes));
            const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
            acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pk[st][qq]), acc_o[dt],
                                                                0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads of the next tile have landed in LDS
    __syncthreads();
  };
  for (int kt = kt0; kt < nkt; kt += 2) {
    key_tile(Stage<0>{}, kt);
    if (kt + 1 < nkt) key_tile(Stage<1>{}, kt + 1);
  }

  // epilogue: lane holds O^T[dims dt*32 + 8 (i/4) + 4 half + (i%4)][its query row]. Each wavefront
  // stages its 32 rows in LDS (both tile buffers are free after the last barrier; 8 KiB per
  // wavefront, 16-byte chunks XOR-swizzled by row) and writes whole 256-byte rows.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (DECODE && chunk_tiles > 0) {
    // partial of chunk blockIdx.z for the G query heads (rows 0 .. G - 1 of wavefront 0): reference max
    // (log2 domain), row sum and unnormalised output, [m, l, -, -, o[128]] per head (16-byte aligned rows)
    if (wave == 0 && col < G) {
      float* pp = part + ((((int64_t)b * hkv + g) * gridDim.z + blockIdx.z) * G + col) * kPartStride;
      if (half == 0) {
        pp[0] = m_ref;
        pp[1] = l_tot;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<f32x4*>(pp + 4 + 32 * dt + 8 * rq + 4 * half) =
              f32x4{acc_o[dt][4 * rq + 0], acc_o[dt][4 * rq + 1], acc_o[dt][4 * rq + 2], acc_o[dt][4 * rq + 3]};
    }
    return;
  }
  if (wave_live) {
    const float inv = 1.f / l_tot;
    char* stage = smem + wave * (32 * kRowBytes);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 w;
        w.x = pack_bf16x2(acc_o[dt][4 * rq + 0] * inv, acc_o[dt][4 * rq + 1] * inv);
        w.y = pack_bf16x2(acc_o[dt][4 * rq + 2] * inv, acc_o[dt][4 * rq + 3] * inv);
        const int chunk = (4 * dt + rq) ^ (col & 15);
        *reinterpret_cast<u32x2*>(stage + col * kRowBytes + 16 * chunk + 8 * half) = w;
      }
    }
    const int p = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 4 * i + (lane >> 4);  // row of the wavefront
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + rr * kRowBytes + 16 * (p ^ (rr & 15)));
      const int rw = wave * 32 + rr;
      const int t = tok_begin + rw / G;
      if (t < tok_end) {
        uint16_t* op = out + ((int64_t)(q0 + t) * hq + g * G + (rw % G)) * kHeadDim + 8 * p;
        // streaming store: nothing in this launch reads the output, so it should not evict the K/V
        // lines that other query tiles of the sequence are about to reuse from L2
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(op));
      }
    }
  }
}

// Merge of the split decode form: out[s, h] = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c over the chunks
// c of sequence s's context that hold keys (M = max_c m_c, the partials' reference maxima in log2 units),
// in chunk order; zero rows for an empty context. One work-group per sequence, 16 lanes of 8 dims per query
// head; the chunks' partials are loaded eight at a time before they are combined.
template <int G>
__global__ __launch_bounds__(1024) void decode_tile_merge_kernel(uint16_t* __restrict__ out,
                                                                 const float* __restrict__ part,
                                                                 const int32_t* __restrict__ context_lens, int hq,
                                                                 int hkv, int max_ctx, int chunks, int chunk_tiles) {
  constexpr int kBatch = 8;
  const int b = blockIdx.x;
  const int h = (int)threadIdx.x >> 4;
  const int d0 = 8 * (threadIdx.x & 15);
  int L = context_lens[b];
  L = L > max_ctx ? max_ctx : L;
  u32x4* op = reinterpret_cast<u32x4*>(out + ((int64_t)b * hq + h) * kHeadDim + d0);
  if (L <= 0) {
    *op = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int nkt = (L + kKeysPerTile - 1) / kKeysPerTile;
  const int nc = (nkt + chunk_tiles - 1) / chunk_tiles;  // chunks that hold keys
  const int g = h / G;
  const float* base = part + (((int64_t)b * hkv + g) * chunks * G + h % G) * kPartStride;
  float M = kNegBig, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += kBatch) {
    float m2[kBatch], l2[kBatch];
    f32x4 lo[kBatch], hi[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + k < nc ? c0 + k : nc - 1;
      const float* pp = base + (int64_t)c * G * kPartStride;
      m2[k] = pp[0];
      l2[k] = pp[1];
      lo[k] = *reinterpret_cast<const f32x4*>(pp + 4 + d0);
      hi[k] = *reinterpret_cast<const f32x4*>(pp + 4 + d0 + 4);
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (c0 + k >= nc) break;
      const float mn = fmaxf(M, m2[k]);
      const float fa = __builtin_amdgcn_exp2f(M - mn);
      const float fb = __builtin_amdgcn_exp2f(m2[k] - mn);
      lsum = lsum * fa + l2[k] * fb;
      const float a2[8] = {lo[k].x, lo[k].y, lo[k].z, lo[k].w, hi[k].x, hi[k].y, hi[k].z, hi[k].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * fa + a2[e] * fb;
      M = mn;
    }
  }
  const float inv = 1.f / lsum;
  u32x4 w;
  w.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *op = w;
}

}  // namespace

}  // namespace pkv

namespace pkv {
namespace {

pkv_status prefill_call(void* out, const void* q, const int32_t* cu_seqlens_q, const int32_t* context_lens,
                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t block_table_stride, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                        int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, float scale, const int32_t* work_items,
                        int32_t num_work_items, void* stream, const NewRows& nr) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0 || num_blocks < 0 ||
      block_table_stride < 0)
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: negative size");
  if (head_dim != kHeadDim)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: head_dim %d (128 only)", head_dim);
  if (block_size != kBlockSize)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: block_size %d (256 only)", block_size);
  if (num_kv_heads < 1 || num_kv_heads > 64 || num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: head counts %d/%d unsupported", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: %d query heads per KV head (1, 2, 4 or 8)", G);
  if (!(scale > 0.f) || !__builtin_isfinite(scale))
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: scale must be finite and > 0");
  if (max_q_len > max_context_len)
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: max_q_len > max_context_len");
  if (num_work_items < 0) return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: num_work_items < 0");
  if (work_items && (reinterpret_cast<uintptr_t>(work_items) & 7))
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: work_items must be 8-byte aligned");
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0 || (work_items && num_work_items == 0)) return ok();
  if (!out || !q || !cu_seqlens_q || !context_lens || !k_cache || !v_cache || !block_tables)
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: q, out and caches must be 16-byte aligned");
  const int64_t need_bt = (max_context_len + kBlockSize - 1) / kBlockSize;
  if (block_table_stride < need_bt)
    return fail(PKV_ERR_INVALID, "paged_attn_prefill_varlen: block_table_stride %d < %lld", block_table_stride,
                (long long)need_bt);
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: more than 65535 sequences");
  const int tok_wg = 128 / G;
  const int ztiles = (max_q_len + tok_wg - 1) / tok_wg;
  if (ztiles > 65535) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_varlen: max_q_len too large");
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid = work_items ? dim3(num_work_items) : dim3(num_kv_heads, num_seqs, ztiles);
  const int2* items = reinterpret_cast<const int2*>(work_items);
  uint16_t* o = static_cast<uint16_t*>(out);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
#define PKV_PREFILL_LAUNCH(GG, FF)                                                                               \
  hipLaunchKernelGGL((prefill_kernel<GG, FF>), grid, dim3(256), 0, s, o, qq, cu_seqlens_q, context_lens, kc, vc, \
                     block_tables, block_table_stride, num_q_heads, num_kv_heads, num_blocks, scale_log2,       \
                     max_q_len, max_context_len, items, num_seqs, nr)
#define PKV_PREFILL_G(FF)                  \
  switch (G) {                             \
    case 1: PKV_PREFILL_LAUNCH(1, FF); break; \
    case 2: PKV_PREFILL_LAUNCH(2, FF); break; \
    case 4: PKV_PREFILL_LAUNCH(4, FF); break; \
    default: PKV_PREFILL_LAUNCH(8, FF); break; \
  }
  if (nr.k) {
    PKV_PREFILL_G(true)
  } else {
    PKV_PREFILL_G(false)
  }
#undef PKV_PREFILL_G
#undef PKV_PREFILL_LAUNCH
  return check_launch("paged_attn_prefill_varlen");
}

}  // namespace
}  // namespace pkv

namespace pkv {

namespace {

template <int G>
pkv_status decode_tile_launch(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int64_t num_blocks,
                              float scale, int32_t max_context_len, void* workspace, size_t workspace_bytes,
                              void* stream, const NewRows& nr) {
  // Split over the keys when the (sequence, KV head) pairs alone would leave the GPU short of work-groups:
  // up to 16 chunks of at least 4 tiles each, aiming at about twice the resident work-groups (three per CU).
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  const int max_tiles = (max_context_len + kKeysPerTile - 1) / kKeysPerTile;
  int chunks = 1;
  if (pairs < kTileDecodeTargetWgs) {
    chunks = (int)((kTileDecodeTargetWgs + pairs - 1) / pairs);
    chunks = chunks < 16 ? chunks : 16;
    const int by_len = max_tiles / 4 > 1 ? max_tiles / 4 : 1;
    chunks = chunks < by_len ? chunks : by_len;
  }
  int chunk_tiles = 0;
  float* part = nullptr;
  if (chunks > 1) {
    chunk_tiles = (max_tiles + chunks - 1) / chunks;
    chunks = (max_tiles + chunk_tiles - 1) / chunk_tiles;
    const size_t need = (size_t)pairs * chunks * G * kPartStride * sizeof(float);
    if (workspace && need <= workspace_bytes && !(reinterpret_cast<uintptr_t>(workspace) & 15)) {
      part = static_cast<float*>(workspace);
    } else {  // not enough workspace for the partials: one work-group per pair
      chunks = 1;
      chunk_tiles = 0;
    }
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(num_kv_heads, num_seqs, chunks);
  uint16_t* o = static_cast<uint16_t*>(out);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);
  if (nr.k)
    hipLaunchKernelGGL((prefill_kernel<G, true, true>), grid, dim3(256), 0, s, o, qq, nullptr, context_lens, kc, vc,
                       block_tables, block_table_stride, num_q_heads, num_kv_heads, num_blocks, scale_log2, 1,
                       max_context_len, nullptr, num_seqs, nr, chunk_tiles, part);
  else
    hipLaunchKernelGGL((prefill_kernel<G, false, true>), grid, dim3(256), 0, s, o, qq, nullptr, context_lens, kc,
                       vc, block_tables, block_table_stride, num_q_heads, num_kv_heads, num_blocks, scale_log2, 1,
                       max_context_len, nullptr, num_seqs, nr, chunk_tiles, part);
  pkv_status st = check_launch("paged_attn_decode (tile form)");
  if (st != PKV_OK || chunks == 1) return st;
  hipLaunchKernelGGL((decode_tile_merge_kernel<G>), dim3(num_seqs), dim3(num_q_heads * 16), 0, s, o, part,
                     context_lens, num_q_heads, num_kv_heads, max_context_len, chunks, chunk_tiles);
  return check_launch("paged_attn_decode (tile form merge)");
}

}  // namespace

pkv_status decode_tile_call(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int64_t num_blocks,
                            float scale, int32_t max_context_len, void* workspace, size_t workspace_bytes,
                            void* stream, const NewRows& nr) {
  if (num_kv_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: head counts %d/%d unsupported", num_q_heads, num_kv_heads);
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: more than 65535 sequences");
  if (num_seqs == 0) return ok();
#define PKV_TILE_DECODE(GG)                                                                                       \
  return decode_tile_launch<GG>(out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs, \
                                num_q_heads, num_kv_heads, num_blocks, scale, max_context_len, workspace,          \
                                workspace_bytes, stream, nr)
  switch (num_q_heads / num_kv_heads) {
    case 2: PKV_TILE_DECODE(2);
    case 4: PKV_TILE_DECODE(4);
    case 8: PKV_TILE_DECODE(8);
    default:
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_decode: the tile form takes 2, 4 or 8 query heads per KV head");
  }
#undef PKV_TILE_DECODE
}

}  // namespace pkv

extern "C" pkv_status paged_attn_prefill_varlen(void* out, const void* q, const int32_t* cu_seqlens_q,
                                                const int32_t* context_lens, const void* k_cache,
                                                const void* v_cache, const int32_t* block_tables,
                                                int32_t block_table_stride, int32_t num_seqs, int32_t total_q,
                                                int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                int64_t num_blocks, float scale, const int32_t* work_items,
                                                int32_t num_work_items, void* stream) {
  const pkv::NewRows none{nullptr, nullptr, 0, 0, nullptr, 0, nullptr, nullptr};
  return pkv::prefill_call(out, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables, block_table_stride,
                           num_seqs, total_q, max_q_len, max_context_len, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, scale, work_items, num_work_items, stream, none);
}

extern "C" pkv_status paged_attn_prefill_store(void* out, const void* q, const void* key, int64_t key_token_stride,
                                               const void* value, int64_t value_token_stride,
                                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                               const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                               const int32_t* block_tables, int32_t block_table_stride,
                                               int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                               int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                               float scale, const int32_t* work_items, int32_t num_work_items,
                                               void* stream) {
  using namespace pkv;
  if (num_seqs > 0 && total_q > 0) {
    if (!key || !value || !slot_mapping) return fail(PKV_ERR_INVALID, "paged_attn_prefill_store: null pointer");
    if (head_dim != kHeadDim)
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_store: head_dim %d (128 only)", head_dim);
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (key_token_stride < row || value_token_stride < row)
      return fail(PKV_ERR_INVALID, "paged_attn_prefill_store: token stride smaller than a row (%lld elements)",
                  (long long)row);
    if ((key_token_stride * 2) % 16 || (value_token_stride * 2) % 16 || !aligned16(key) || !aligned16(value))
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_store: key/value and their strides must be 16-byte aligned");
    if (key_token_stride > (1 << 25) || value_token_stride > (1 << 25))
      return fail(PKV_ERR_UNSUPPORTED, "paged_attn_prefill_store: token stride above 2^25 elements");
    if (num_blocks > INT64_MAX / kBlockSize)
      return fail(PKV_ERR_INVALID, "paged_attn_prefill_store: num_blocks out of range");
  }
  const NewRows nr{static_cast<const char*>(key), static_cast<const char*>(value), key_token_stride * 2,
                   value_token_stride * 2, slot_mapping, num_blocks * kBlockSize, static_cast<char*>(k_cache),
                   static_cast<char*>(v_cache)};
  return prefill_call(out, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables, block_table_stride,
                      num_seqs, total_q, max_q_len, max_context_len, num_q_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, scale, work_items, num_work_items, stream, nr);
}
