// Host side of the C ABI: error reporting and the per-step metadata builder.
//
// Page reference: P1 = "13. 读一个最小推理引擎：nano-vllm".

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <string>
#include <vector>

#include "common.h"

namespace pkv {

static thread_local std::string g_error;

pkv_status fail(pkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

pkv_status ok() {
  g_error.clear();
  return PKV_OK;
}

pkv_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_error.c_str(); }

extern "C" int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

// Step preparation (P1, "第五站：执行准备与 KV 容量"): one slot per token the
// step computes, positions num_cached .. seq_len - 1 of each sequence
// (P1, "第二站"), slot = table[pos / bs] * bs + pos % bs; padding rows get -1.
extern "C" pkv_status pkv_prepare_step(int32_t num_seqs, const int32_t* seq_lens,
                                       const int32_t* num_cached, const int32_t* bt_data,
                                       const int64_t* bt_off, int32_t num_pad, int32_t block_size,
                                       int32_t max_blocks_per_seq, int32_t* out_slots,
                                       int64_t slot_capacity, int32_t* out_cu, int32_t* out_ctx,
                                       int32_t* out_bt, int64_t* out_num_tokens,
                                       int32_t* out_max_q, int32_t* out_max_ctx) {
  using pkv::fail;
  if (num_seqs < 0 || num_pad < 0) return fail(PKV_ERR_INVALID, "pkv_prepare_step: negative count");
  if (block_size <= 0) return fail(PKV_ERR_INVALID, "pkv_prepare_step: block_size must be > 0");
  if (max_blocks_per_seq < 0) return fail(PKV_ERR_INVALID, "pkv_prepare_step: max_blocks_per_seq < 0");
  if (slot_capacity < 0) return fail(PKV_ERR_INVALID, "pkv_prepare_step: slot_capacity < 0");
  const int64_t rows = (int64_t)num_seqs + num_pad;
  if (!out_cu || !out_ctx || (rows > 0 && max_blocks_per_seq > 0 && !out_bt))
    return fail(PKV_ERR_INVALID, "pkv_prepare_step: null output pointer");
  if (num_seqs > 0 && (!seq_lens || !num_cached || !bt_off))
    return fail(PKV_ERR_INVALID, "pkv_prepare_step: null input pointer");
  // validate everything before writing anything
  int64_t total = num_pad;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = seq_lens[s], c = num_cached[s];
    if (L < 1 || c < 0 || c >= L)
      return fail(PKV_ERR_INVALID, "pkv_prepare_step: seq %d needs 0 <= num_cached < seq_len (got %lld, %lld)",
                  s, (long long)c, (long long)L);
    const int64_t nb = bt_off[s + 1] - bt_off[s];
    const int64_t need = (L + block_size - 1) / block_size;
    if (nb < need || nb > max_blocks_per_seq)
      return fail(PKV_ERR_INVALID, "pkv_prepare_step: seq %d has %lld blocks, needs %lld (max %d)", s,
                  (long long)nb, (long long)need, max_blocks_per_seq);
    if (nb > 0 && !bt_data) return fail(PKV_ERR_INVALID, "pkv_prepare_step: null block_table_data");
    for (int64_t j = 0; j < nb; ++j) {
      const int64_t blk = bt_data[bt_off[s] + j];
      if (blk < 0) return fail(PKV_ERR_INVALID, "pkv_prepare_step: seq %d block %lld is negative", s, (long long)j);
      if ((blk + 1) * (int64_t)block_size - 1 > INT32_MAX)
        return fail(PKV_ERR_INVALID, "pkv_prepare_step: seq %d block %lld: slot exceeds int32", s, (long long)j);
    }
    total += L - c;
  }
  if (total > slot_capacity || (total > 0 && !out_slots))
    return fail(PKV_ERR_INVALID, "pkv_prepare_step: %lld slots needed, capacity %lld", (long long)total,
                (long long)slot_capacity);
  if (total > INT32_MAX) return fail(PKV_ERR_INVALID, "pkv_prepare_step: token count exceeds int32");

  int64_t t = 0;
  int32_t max_q = 0, max_ctx = 0;
  out_cu[0] = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s], c = num_cached[s];
    const int32_t* table = bt_data + bt_off[s];
    for (int32_t pos = c; pos < L; ++pos)
      out_slots[t++] = table[pos / block_size] * block_size + pos % block_size;
    out_cu[s + 1] = (int32_t)t;
    out_ctx[s] = L;
    const int64_t nb = bt_off[s + 1] - bt_off[s];
    int32_t* row = out_bt + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nb ? table[j] : -1;
    if (L - c > max_q) max_q = L - c;
    if (L > max_ctx) max_ctx = L;
  }
  for (int32_t p = 0; p < num_pad; ++p) {
    out_slots[t++] = -1;
    out_cu[num_seqs + p + 1] = (int32_t)t;
    out_ctx[num_seqs + p] = 0;
    int32_t* row = out_bt + ((int64_t)num_seqs + p) * max_blocks_per_seq;
    for (int64_t j = 0; j < max_blocks_per_seq; ++j) row[j] = -1;
    if (max_q < 1) max_q = 1;
  }
  if (out_num_tokens) *out_num_tokens = t;
  if (out_max_q) *out_max_q = max_q;
  if (out_max_ctx) *out_max_ctx = max_ctx;
  return pkv::ok();
}

// Prefill work list: one item per (sequence, query tile, KV head) that holds
// at least one query token, heaviest first. An item's cost is the number of
// 64-key tiles it reads (its last query sits at c + tile_end - 1), so the
// long items start first and the short ones fill the tail of the launch.
// Within equal cost the order is sequence, later tile first, KV head, which
// keeps the KV heads of one (sequence, tile) adjacent: with round-robin
// dispatch over the XCDs every tile of one KV head then meets the same L2.
extern "C" pkv_status pkv_prefill_plan(int32_t num_seqs, const int32_t* cu_seqlens_q,
                                       const int32_t* context_lens, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t* out_items, int64_t capacity,
                                       int64_t* out_num_items) {
  using pkv::fail;
  if (num_seqs < 0 || capacity < 0) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: negative size");
  if (!out_num_items) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: null out_num_items");
  if (num_kv_heads < 1 || num_kv_heads > 64 || num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_prefill_plan: head counts %d/%d unsupported", num_q_heads, num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_prefill_plan: %d query heads per KV head (1, 2, 4 or 8)", G);
  if (num_seqs > 0 && (!cu_seqlens_q || !context_lens))
    return fail(PKV_ERR_INVALID, "pkv_prefill_plan: null input pointer");
  const int tok_wg = 128 / G;  // query tokens per work-group of the prefill kernel
  int64_t count = 0;
  if (num_seqs > 0 && cu_seqlens_q[0] != 0) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: cu_seqlens_q[0] != 0");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    const int64_t L = context_lens[s];
    if (n < 0) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: cu_seqlens_q decreases at %d", s);
    if (L < n) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: seq %d context %lld < %lld query tokens", s,
                           (long long)L, (long long)n);
    if (n > ((int64_t)1 << 23) * tok_wg)
      return fail(PKV_ERR_UNSUPPORTED, "pkv_prefill_plan: seq %d has more than 2^23 query tiles", s);
    count += ((n + tok_wg - 1) / tok_wg) * num_kv_heads;
  }
  if (count > INT32_MAX) return fail(PKV_ERR_INVALID, "pkv_prefill_plan: more than 2^31 - 1 items");
  *out_num_items = count;
  if (!out_items) return pkv::ok();  // size query
  if (count > capacity)
    return fail(PKV_ERR_INVALID, "pkv_prefill_plan: %lld items, capacity %lld", (long long)count,
                (long long)capacity);
  struct Tile {
    int64_t cost;
    int32_t seq, tile;
  };
  std::vector<Tile> tiles;
  tiles.reserve(count / num_kv_heads);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
    const int64_t c = context_lens[s] - n;
    for (int64_t t = (n + tok_wg - 1) / tok_wg - 1; t >= 0; --t) {
      const int64_t end = (t + 1) * tok_wg < n ? (t + 1) * tok_wg : n;
      tiles.push_back({(c + end + 63) / 64, s, (int32_t)t});
    }
  }
  std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& x, const Tile& y) { return x.cost > y.cost; });
  int64_t at = 0;
  for (const Tile& t : tiles)
    for (int32_t g = 0; g < num_kv_heads; ++g, ++at) {
      out_items[2 * at] = t.seq;
      out_items[2 * at + 1] = (t.tile << 8) | g;
    }
  return pkv::ok();
}
