// Host-side C ABI under AddressSanitizer / UndefinedBehaviorSanitizer: drives
// the step preparation, the prefill work plan, the scheduler and the graph
// argument checks with valid and malformed inputs. Built (host code only)
// and run by tests/test_asan_host.py; exits non-zero on a failed check, and
// the sanitizers abort on any invalid memory access.

#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "pkv.h"

namespace pkv {
// graph.cpp calls into the decode library only after its argument checks;
// these stand-ins end the run if that is ever reached here
bool decode_prepare(int32_t, int32_t, int32_t) {
  fprintf(stderr, "decode_prepare reached\n");
  abort();
}
}  // namespace pkv

extern "C" pkv_status paged_attn_decode_store(void*, const void*, const void*, int64_t, const void*, int64_t,
                                              const int32_t*, void*, void*, const int32_t*, int32_t,
                                              const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int64_t,
                                              float, int32_t, void*, size_t, void*) {
  fprintf(stderr, "paged_attn_decode_store reached\n");
  abort();
}

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static void prepare_step(std::mt19937& rng) {
  for (int trial = 0; trial < 300; ++trial) {
    const int S = (int)(rng() % 40), pad = (int)(rng() % 5), bs = 1 << (rng() % 9), mb = 1 + (int)(rng() % 12);
    std::vector<int32_t> lens(S), cached(S), data;
    std::vector<int64_t> offs(S + 1, 0);
    int64_t T = pad;
    for (int s = 0; s < S; ++s) {
      const int nb = 1 + (int)(rng() % mb);
      lens[s] = 1 + (int)(rng() % (nb * bs));
      cached[s] = (int)(rng() % lens[s]);
      const int need = (lens[s] + bs - 1) / bs;
      for (int j = 0; j < need; ++j) data.push_back((int32_t)(rng() % 1000));
      offs[s + 1] = (int64_t)data.size();
      T += lens[s] - cached[s];
    }
    const bool short_cap = (rng() % 7) == 0;
    std::vector<int32_t> slots(T + 1), cu(S + pad + 1), ctx(S + pad + 1), bt((size_t)(S + pad) * mb + 1);
    int64_t nt = -1;
    int32_t mq = -1, mc = -1;
    const pkv_status st = pkv_prepare_step(S, lens.data(), cached.data(), data.empty() ? nullptr : data.data(),
                                           offs.data(), pad, bs, mb, slots.data(), short_cap ? T - 1 : T, cu.data(),
                                           ctx.data(), bt.data(), &nt, &mq, &mc);
    if (short_cap && T > 0) {
      CHECK(st == PKV_ERR_INVALID);
      continue;
    }
    CHECK(st == PKV_OK);
    CHECK(nt == T);
    for (int s = 0; s < S; ++s)
      for (int p = cached[s], i = (int)cu[s]; p < lens[s]; ++p, ++i)
        CHECK(slots[i] == data[offs[s] + p / bs] * bs + p % bs);
  }
  // malformed: a table shorter than the sequence, negative cached, a null output
  int32_t L[1] = {600}, C[1] = {0}, D[2] = {1, 2}, out[700], cu[2], ctx[1], btab[4];
  int64_t O[2] = {0, 2};
  CHECK(pkv_prepare_step(1, L, C, D, O, 0, 256, 4, out, 700, cu, ctx, btab, nullptr, nullptr, nullptr) ==
        PKV_ERR_INVALID);
  C[0] = -1;
  L[0] = 300;
  CHECK(pkv_prepare_step(1, L, C, D, O, 0, 256, 4, out, 700, cu, ctx, btab, nullptr, nullptr, nullptr) ==
        PKV_ERR_INVALID);
  C[0] = 0;
  CHECK(pkv_prepare_step(1, L, C, D, O, 0, 256, 4, nullptr, 700, cu, ctx, btab, nullptr, nullptr, nullptr) !=
        PKV_OK);
  CHECK(pkv_prepare_step(1, L, C, D, O, 0, 256, 1, out, 700, cu, ctx, btab, nullptr, nullptr, nullptr) ==
        PKV_ERR_INVALID);  // stride smaller than the table
}

static void prefill_plan(std::mt19937& rng) {
  const int heads[][2] = {{16, 8}, {8, 8}, {32, 8}, {64, 8}, {4, 1}};
  for (int trial = 0; trial < 300; ++trial) {
    const int S = (int)(rng() % 50);
    std::vector<int32_t> cu(S + 1, 0), ctx(S + 1);
    for (int s = 0; s < S; ++s) {
      cu[s + 1] = cu[s] + (int)(rng() % 700);
      ctx[s] = cu[s + 1] - cu[s] + (int)(rng() % 600);
    }
    const int* h = heads[rng() % 5];
    int64_t n = -1;
    CHECK(pkv_prefill_plan(S, cu.data(), ctx.data(), h[0], h[1], nullptr, 0, &n) == PKV_OK);
    std::vector<int32_t> items(2 * (size_t)n + 2);
    if (n > 0) {
      int64_t m = -1;
      CHECK(pkv_prefill_plan(S, cu.data(), ctx.data(), h[0], h[1], items.data(), n - 1, &m) == PKV_ERR_INVALID);
    }
    int64_t m = -1;
    CHECK(pkv_prefill_plan(S, cu.data(), ctx.data(), h[0], h[1], items.data(), n, &m) == PKV_OK && m == n);
    for (int64_t i = 0; i < n; ++i) CHECK(items[2 * i] >= 0 && items[2 * i] < S && (items[2 * i + 1] & 255) < h[1]);
  }
  int32_t cu[3] = {0, 5, 3}, ctx[2] = {5, 9};
  int64_t n;
  CHECK(pkv_prefill_plan(2, cu, ctx, 16, 8, nullptr, 0, &n) == PKV_ERR_INVALID);  // decreasing
  cu[2] = 9;
  ctx[1] = 3;
  CHECK(pkv_prefill_plan(2, cu, ctx, 16, 8, nullptr, 0, &n) == PKV_ERR_INVALID);  // context shorter than the run
  CHECK(pkv_prefill_plan(2, cu, ctx, 24, 8, nullptr, 0, &n) == PKV_ERR_UNSUPPORTED);
  CHECK(pkv_prefill_plan(2, nullptr, ctx, 16, 8, nullptr, 0, &n) == PKV_ERR_INVALID);
}

static void scheduler(std::mt19937& rng) {
  for (int trial = 0; trial < 60; ++trial) {
    const int blocks = 4 + (int)(rng() % 60), bs = 1 << (2 + rng() % 7);
    pkv_sched* s = nullptr;
    CHECK(pkv_sched_create(blocks, bs, 1 + (int)(rng() % 16), 16 + (int)(rng() % 2000), &s) == PKV_OK);
    const int nreq = 1 + (int)(rng() % 30);
    for (int r = 0; r < nreq; ++r) {
      const int p = 1 + (int)(rng() % (bs * 3)), o = 1 + (int)(rng() % (bs * 2));
      CHECK(pkv_sched_add(s, p, o, nullptr) == PKV_OK);
    }
    for (int step = 0; step < 100000; ++step) {
      pkv_sched_batch b;
      const pkv_status st = pkv_sched_schedule(s, &b);
      if (st != PKV_OK) break;  // a request larger than the pool: reported, not run
      if (b.kind == PKV_STEP_NONE) break;
      CHECK(pkv_sched_schedule(s, &b) == PKV_ERR_INVALID);   // must postprocess first
      CHECK(pkv_sched_add(s, 5, 5, nullptr) == PKV_ERR_INVALID);
      int64_t used = 0;
      for (int i = 0; i < b.num_seqs; ++i) {
        CHECK(b.num_cached[i] >= 0 && b.num_cached[i] < b.seq_lens[i]);
        const int64_t nb = b.bt_offsets[i + 1] - b.bt_offsets[i];
        CHECK(nb * bs >= b.seq_lens[i]);
        for (int64_t j = b.bt_offsets[i]; j < b.bt_offsets[i + 1]; ++j) CHECK(b.bt_data[j] >= 0 && b.bt_data[j] < blocks);
        used += nb;
      }
      CHECK(used + pkv_sched_free_blocks(s) <= blocks);
      for (int i = 0; i < b.num_preempted; ++i) CHECK(b.preempted[i] >= 0 && b.preempted[i] < nreq);
      CHECK(pkv_sched_postprocess(s) == PKV_OK);
    }
    CHECK(pkv_sched_destroy(s) == PKV_OK);
  }
  pkv_sched* s = nullptr;
  CHECK(pkv_sched_create(0, 256, 4, 100, nullptr) == PKV_ERR_INVALID);
  CHECK(pkv_sched_create(8, 0, 4, 100, &s) == PKV_ERR_INVALID);
  CHECK(pkv_sched_add(nullptr, 1, 1, nullptr) == PKV_ERR_INVALID);
  CHECK(pkv_sched_unfinished(nullptr) == -1 && pkv_sched_free_blocks(nullptr) == -1);
  CHECK(pkv_sched_create(2, 16, 4, 100, &s) == PKV_OK);
  CHECK(pkv_sched_add(s, 100, 3, nullptr) == PKV_OK);  // needs 7 blocks of a 2-block pool
  pkv_sched_batch b;
  CHECK(pkv_sched_schedule(s, &b) == PKV_ERR_INVALID);
  CHECK(pkv_sched_destroy(s) == PKV_OK);
}

static void graphs() {
  pkv_decode_graph_desc d{};
  pkv_decode_graphs* g = nullptr;
  const int32_t good[3] = {1, 2, 4}, bad[3] = {1, 4, 2};
  CHECK(pkv_decode_graphs_create(&d, good, 3, nullptr) == PKV_ERR_INVALID);
  CHECK(pkv_decode_graphs_create(nullptr, good, 3, &g) == PKV_ERR_INVALID && g == nullptr);
  CHECK(pkv_decode_graphs_create(&d, bad, 3, &g) == PKV_ERR_INVALID && g == nullptr);
  CHECK(pkv_decode_graphs_create(&d, good, 0, &g) == PKV_ERR_INVALID);
  CHECK(pkv_decode_graphs_create_layers(&d, 0, good, 3, &g) == PKV_ERR_INVALID);
  CHECK(pkv_decode_graphs_launch(nullptr, 1, nullptr, nullptr) == PKV_ERR_INVALID);
  CHECK(pkv_decode_graphs_destroy(nullptr) == PKV_OK);
}

int main() {
  std::mt19937 rng(12345);
  prepare_step(rng);
  prefill_plan(rng);
  scheduler(rng);
  graphs();
  CHECK(pkv_last_error() != nullptr);
  printf("host driver: %d failed checks\n", failures);
  return failures ? 1 : 0;
}
