// Native scheduler and block manager (host): which sequences run in a step and
// which cache blocks they own.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm".
//  * "第三站：调度器": a step first tries prefill, taking waiting requests in
//    FCFS order within max_num_seqs, the token budget and the free blocks;
//    only the first request of a step may be cut to the remaining budget (it
//    stays at the head of the waiting queue); any prefill makes the step
//    prefill-only. Otherwise every running sequence advances one token; when
//    blocks run out the most recently added running sequence is preempted,
//    frees its blocks and returns to the front of the waiting queue to be
//    recomputed.
//  * "第四站：块管理与前缀缓存": first scheduling allocates blocks for the
//    whole current length; a decode step needs a new block exactly when
//    len % block_size == 1; freed blocks return to a FIFO free queue. Prefix
//    caching needs token ids and is not part of this token-free scheduler.
//  * "第五站：执行准备与 KV 容量": decode batches are padded up to a replay
//    bucket (1, 2, 4, 8, then multiples of 16 up to 512).
//  * "第一站：主循环": a completed prompt yields one token, each decode step
//    one token; a request finishes after its output length.
// Where the pages leave a step open: O output tokens take O - 1 decode steps;
// a chunk yields nothing until the prompt is complete; a preempted request
// re-prefills from position 0; allocation takes from the front of the free
// queue and release appends in table order; victims come from the back of
// the running list until the sequence being extended has a block (itself if
// it is the newest left); a request longer than the whole pool is an error.

#include <deque>
#include <new>
#include <vector>

#include "common.h"

struct pkv_sched {
  struct Req {
    int32_t prompt_len = 0, output_len = 0, generated = 0, num_cached = 0;
    std::vector<int32_t> blocks;
    bool done = false;
    int32_t length() const { return prompt_len + generated; }
  };
  int32_t block_size = 0, max_num_seqs = 0, budget = 0, num_blocks = 0;
  std::deque<int32_t> free_blocks;
  std::vector<Req> reqs;
  std::deque<int32_t> waiting;   // request ids
  std::vector<int32_t> running;  // request ids, in the order they were added
  int32_t unfinished = 0;

  // the batch of the last schedule() call, until postprocess()
  bool pending = false;
  int32_t kind = -1;
  std::vector<int32_t> b_ids, b_ntok, b_lens, b_cached, b_full, b_bt, b_pre;
  std::vector<int64_t> b_off;
  int32_t b_pad = 0, b_chunked = 0;

  int32_t need(int32_t len) const { return (len + block_size - 1) / block_size; }
  void release(Req& r) {
    for (int32_t blk : r.blocks) free_blocks.push_back(blk);
    r.blocks.clear();
  }
  void take(Req& r, int32_t n) {
    for (int32_t i = 0; i < n; ++i) {
      r.blocks.push_back(free_blocks.front());
      free_blocks.pop_front();
    }
  }
  static int32_t bucket(int32_t n) {
    if (n <= 8) return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8;
    if (n <= 512) return (n + 15) / 16 * 16;
    return n;
  }
  void record(int32_t id, int32_t len, int32_t cached) {
    const Req& r = reqs[id];
    b_ids.push_back(id);
    b_lens.push_back(len);
    b_cached.push_back(cached);
    b_full.push_back(r.length());
    b_bt.insert(b_bt.end(), r.blocks.begin(), r.blocks.end());
    b_off.push_back((int64_t)b_bt.size());
  }
  void clear_batch() {
    b_ids.clear(); b_ntok.clear(); b_lens.clear(); b_cached.clear(); b_full.clear(); b_bt.clear(); b_pre.clear();
    b_off.assign(1, 0);
    b_pad = 0;
    b_chunked = 0;
    kind = -1;
  }

  // prefill phase; true when something was scheduled
  bool try_prefill() {
    int32_t tokens = 0;
    while (!waiting.empty() && (int32_t)running.size() + (int32_t)b_ids.size() < max_num_seqs) {
      Req& r = reqs[waiting.front()];
      const int32_t remaining = budget - tokens;
      const int32_t todo = r.length() - r.num_cached;
      if (remaining < todo && !b_ids.empty()) break;
      if (r.blocks.empty()) {
        if ((int32_t)free_blocks.size() < need(r.length())) break;
        take(r, need(r.length()));
      }
      const int32_t n = todo < remaining ? todo : remaining;
      if (n <= 0) break;
      record(waiting.front(), r.num_cached + n, r.num_cached);
      b_ntok.push_back(n);
      tokens += n;
      if (n < todo) {
        b_chunked = 1;
        break;  // the remainder stays at the head of the waiting queue
      }
      waiting.pop_front();
    }
    return !b_ids.empty();
  }

  // decode phase: extend every running sequence by one token, preempting
  // the newest ones when no block is free
  void decode() {
    std::deque<int32_t> queue(running.begin(), running.end());
    running.clear();
    while (!queue.empty()) {
      const int32_t id = queue.front();
      queue.pop_front();
      Req& r = reqs[id];
      bool ok = true;
      while (r.length() % block_size == 1 && free_blocks.empty()) {
        int32_t victim;
        if (!queue.empty()) {
          victim = queue.back();
          queue.pop_back();
        } else {
          ok = false;  // r is the newest one left
          victim = id;
        }
        Req& v = reqs[victim];
        release(v);
        v.num_cached = 0;
        waiting.push_front(victim);
        b_pre.push_back(victim);
        if (!ok) break;
      }
      if (!ok) break;
      if (r.length() % block_size == 1) take(r, 1);
      running.push_back(id);
    }
    for (int32_t id : running) record(id, reqs[id].length(), reqs[id].length() - 1);
  }
};

namespace {

pkv_status check(const pkv_sched* s, const char* fn) {
  if (!s) return pkv::fail(PKV_ERR_INVALID, "%s: null scheduler", fn);
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t max_num_seqs,
                                       int32_t max_num_batched_tokens, pkv_sched** out) {
  using pkv::fail;
  if (!out) return fail(PKV_ERR_INVALID, "pkv_sched_create: null output");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0 || max_num_seqs <= 0 || max_num_batched_tokens <= 0)
    return fail(PKV_ERR_INVALID, "pkv_sched_create: sizes must be positive (blocks >= 0)");
  pkv_sched* s = new (std::nothrow) pkv_sched;
  if (!s) return fail(PKV_ERR_INVALID, "pkv_sched_create: out of host memory");
  s->num_blocks = num_blocks;
  s->block_size = block_size;
  s->max_num_seqs = max_num_seqs;
  s->budget = max_num_batched_tokens;
  for (int32_t b = 0; b < num_blocks; ++b) s->free_blocks.push_back(b);
  s->clear_batch();
  *out = s;
  return pkv::ok();
}

extern "C" pkv_status pkv_sched_destroy(pkv_sched* s) {
  delete s;
  return pkv::ok();
}

extern "C" pkv_status pkv_sched_add(pkv_sched* s, int32_t prompt_len, int32_t output_len, int32_t* out_id) {
  using pkv::fail;
  if (pkv_status st = check(s, "pkv_sched_add")) return st;
  if (prompt_len < 1 || output_len < 1)
    return fail(PKV_ERR_INVALID, "pkv_sched_add: prompt and output lengths must be >= 1");
  if ((int64_t)prompt_len + output_len - 1 > INT32_MAX)
    return fail(PKV_ERR_INVALID, "pkv_sched_add: total length exceeds int32");
  if (s->pending) return fail(PKV_ERR_INVALID, "pkv_sched_add: a scheduled step awaits pkv_sched_postprocess");
  pkv_sched::Req r;
  r.prompt_len = prompt_len;
  r.output_len = output_len;
  s->reqs.push_back(r);
  const int32_t id = (int32_t)s->reqs.size() - 1;
  s->waiting.push_back(id);
  ++s->unfinished;
  if (out_id) *out_id = id;
  return pkv::ok();
}

extern "C" pkv_status pkv_sched_schedule(pkv_sched* s, pkv_sched_batch* out) {
  using pkv::fail;
  if (pkv_status st = check(s, "pkv_sched_schedule")) return st;
  if (!out) return fail(PKV_ERR_INVALID, "pkv_sched_schedule: null output");
  if (s->pending) return fail(PKV_ERR_INVALID, "pkv_sched_schedule: previous step not postprocessed");
  s->clear_batch();
  for (;;) {
    if (s->waiting.empty() && s->running.empty()) break;  // nothing left: kind stays -1
    if (s->try_prefill()) {
      s->kind = 1;
      break;
    }
    if (s->running.empty()) {
      // nothing runs and the head of the queue cannot start: it needs more
      // blocks than the pool holds (or max_num_seqs is exhausted by nothing)
      return fail(PKV_ERR_INVALID, "pkv_sched_schedule: request %d needs %d blocks, pool has %d free of %d",
                  s->waiting.front(), s->need(s->reqs[s->waiting.front()].length()),
                  (int)s->free_blocks.size(), s->num_blocks);
    }
    s->decode();
    if (!s->b_ids.empty()) {
      s->kind = 0;
      s->b_pad = pkv_sched::bucket((int32_t)s->b_ids.size()) - (int32_t)s->b_ids.size();
      break;
    }
    // every running sequence was preempted: try again (prefill first)
    const std::vector<int32_t> pre = s->b_pre;
    s->clear_batch();
    s->b_pre = pre;
  }
  s->pending = s->kind >= 0;
  out->kind = s->kind;
  out->num_seqs = (int32_t)s->b_ids.size();
  out->num_pad = s->b_pad;
  out->chunked_first = s->b_chunked;
  out->num_preempted = (int32_t)s->b_pre.size();
  out->request_ids = s->b_ids.data();
  out->seq_lens = s->b_lens.data();
  out->num_cached = s->b_cached.data();
  out->full_lens = s->b_full.data();
  out->bt_offsets = s->b_off.data();
  out->bt_data = s->b_bt.data();
  out->preempted = s->b_pre.data();
  return pkv::ok();
}

extern "C" pkv_status pkv_sched_postprocess(pkv_sched* s) {
  using pkv::fail;
  if (pkv_status st = check(s, "pkv_sched_postprocess")) return st;
  if (!s->pending) return fail(PKV_ERR_INVALID, "pkv_sched_postprocess: no scheduled step");
  s->pending = false;
  auto finish = [&](pkv_sched::Req& r) {
    r.done = true;
    s->release(r);
    --s->unfinished;
  };
  if (s->kind == 1) {
    for (size_t i = 0; i < s->b_ids.size(); ++i) {
      pkv_sched::Req& r = s->reqs[s->b_ids[i]];
      r.num_cached += s->b_ntok[i];
      if (r.num_cached == r.length()) {  // prompt complete: one token out
        s->running.push_back(s->b_ids[i]);
        r.generated += 1;
        if (r.generated >= r.output_len) {
          s->running.pop_back();
          finish(r);
        }
      }
    }
  } else {
    std::vector<int32_t> still;
    for (int32_t id : s->running) {
      pkv_sched::Req& r = s->reqs[id];
      r.num_cached = r.length();
      r.generated += 1;
    }
    for (int32_t id : s->running) {
      pkv_sched::Req& r = s->reqs[id];
      if (r.generated >= r.output_len) finish(r);
      else still.push_back(id);
    }
    s->running.swap(still);
  }
  return pkv::ok();
}

extern "C" int32_t pkv_sched_unfinished(const pkv_sched* s) { return s ? s->unfinished : -1; }

extern "C" int32_t pkv_sched_free_blocks(const pkv_sched* s) { return s ? (int32_t)s->free_blocks.size() : -1; }
