"""Plain Python scheduler and block manager: the oracle for the native scheduler.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and
the CPU-baseline leg of the benchmark may call this module.

A token-free simulation of the engine loop the pages describe. Each step it
decides which sequences run and which blocks they own, and it records every
sequence's state (length after the step, tokens already cached, block table).
It computes no slot and no attention: the step's metadata follows from those
states (``paged.prepare_step_ref``).

Page references, P1 = "13. 读一个最小推理引擎：nano-vllm":

* "第三站：调度器": a step first tries prefill, taking waiting requests in FCFS
  order while the number of running sequences stays within max_num_seqs, the
  token budget (max_num_batched_tokens) has room and enough free blocks
  exist; only the first request of a step may be cut to the remaining budget
  (its remainder stays at the head of the waiting queue); any prefill makes
  the step prefill-only. Otherwise every running sequence advances one token;
  when blocks run out, the most recently added running sequence is preempted:
  it frees all its blocks and goes back to the front of the waiting queue, to
  be recomputed (no swap to host).
* "第四站：块管理与前缀缓存": a request scheduled for the first time gets
  blocks for its whole current length at once; a decode step needs a new
  block exactly when len(seq) % block_size == 1; freed blocks return to the
  free queue. Prefix caching hashes token ids, which token-free requests do
  not have, so it is off.
* "第五站：执行准备与 KV 容量": decode batches are padded up to a replay
  bucket (1, 2, 4, 8, then multiples of 16 up to 512).
* "第一站：主循环": a prefill that completes a prompt yields one token; each
  decode step yields one token; a request finishes after output_len tokens.

Readings (where the pages leave a step open):
* a request with output length O therefore runs O - 1 decode steps, and the
  K/V of its final token is never stored;
* a chunked prefill yields no token until its last chunk;
* after a preemption the request re-prefills its prompt plus the tokens
  generated so far, from position 0;
* the free-block queue is FIFO: allocation takes from the front, release
  appends the blocks in table order;
* preemption victims are taken from the back of the running list (newest
  first) until the sequence being extended has a block, and that sequence is
  preempted itself when it is the newest one left;
* within one decode step, sequences are extended in running order, and a
  sequence preempted while the batch forms does not run in that step; when
  every running sequence is preempted no decode step is recorded, and the
  preemptions are reported with the next recorded step;
* a request that needs more blocks than the whole pool is an error (the
  schedule could never run it).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

from workloads import Batch, Seq

BUCKETS = [1, 2, 4, 8] + list(range(16, 513, 16))


@dataclass
class Request:
    rid: int
    prompt_len: int
    output_len: int
    generated: int = 0
    num_cached: int = 0
    block_table: list = field(default_factory=list)
    done: bool = False

    @property
    def length(self) -> int:
        return self.prompt_len + self.generated


@dataclass
class TraceStep:
    index: int
    kind: str            # "prefill" or "decode"
    batch: Batch         # sequence states for this step (block tables copied)
    preempted: list      # request ids preempted while forming this step
    chunked_first: bool  # the first prefill sequence was cut to the budget
    rids: list           # request id of each sequence in the batch
    full_lens: list      # each sequence's whole length (prompt + generated) at this step


class BlockPool:
    """Free-block FIFO with one owner per block (no sharing without prefix
    caching)."""

    def __init__(self, num_blocks: int):
        self.free = deque(range(num_blocks))
        self.num_blocks = num_blocks

    def allocate(self, n: int) -> list:
        assert len(self.free) >= n
        return [self.free.popleft() for _ in range(n)]

    def release(self, blocks):
        self.free.extend(blocks)


def bucket(n: int) -> int:
    """Smallest replay bucket holding n rows (n itself above the largest)."""
    for b in BUCKETS:
        if b >= n:
            return b
    return n


def replay(prompts, outputs, num_blocks: int, max_num_seqs: int, budget: int, block_size: int = 256):
    """Run the schedule to completion; returns (steps, requests, pool)."""
    reqs = [Request(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]
    waiting = deque(reqs)
    running: list = []   # in the order sequences were added
    pool = BlockPool(num_blocks)
    steps = []
    need = lambda L: -(-L // block_size)  # noqa: E731
    carried: list = []   # preemptions of a decode phase that recorded no step

    while waiting or running:
        # ---- prefill phase ----
        scheduled, tokens, chunked = [], 0, False
        while waiting and len(running) + len(scheduled) < max_num_seqs:
            r = waiting[0]
            remaining = budget - tokens
            todo = r.length - r.num_cached
            if remaining < todo and scheduled:
                break
            if not r.block_table:
                if len(pool.free) < need(r.length):
                    break
                r.block_table = pool.allocate(need(r.length))
            n = min(todo, remaining)
            if n <= 0:
                break
            scheduled.append((r, n))
            tokens += n
            if n < todo:
                chunked = True
                break           # stays at the head of waiting
            waiting.popleft()
        if scheduled:
            seqs = [Seq(r.num_cached + n, r.num_cached, list(r.block_table)) for r, n in scheduled]
            steps.append(TraceStep(len(steps), "prefill", Batch(seqs, 0, stream=len(steps)), carried, chunked,
                                   [r.rid for r, _ in scheduled], [r.length for r, _ in scheduled]))
            carried = []
            for r, n in scheduled:
                r.num_cached += n
                if r.num_cached == r.length:          # prompt complete: one token out
                    running.append(r)
                    r.generated += 1
                    if r.generated >= r.output_len:
                        r.done = True
                        running.remove(r)
                        pool.release(r.block_table)
                        r.block_table = []
            continue
        if not running:
            raise ValueError(f"request {waiting[0].rid} needs {need(waiting[0].length)} blocks; "
                             f"the pool has {num_blocks}")
        # ---- decode phase ----
        preempted, batch = carried, []
        carried = []
        queue = list(running)
        running = []
        while queue:
            r = queue.pop(0)
            # the token at position length - 1 opens a new block when length % bs == 1
            ok = True
            while (r.length % block_size == 1) and not pool.free:
                victim = queue.pop() if queue else None
                if victim is None:               # r is the newest left: preempt it
                    ok = False
                    victim = r
                pool.release(victim.block_table)
                victim.block_table = []
                victim.num_cached = 0
                waiting.appendleft(victim)
                preempted.append(victim.rid)
                if not ok:
                    break
            if not ok:
                break
            if r.length % block_size == 1:
                r.block_table += pool.allocate(1)
            batch.append(r)
        running = batch
        if not batch:
            carried = preempted
            continue
        seqs = [Seq(r.length, r.length - 1, list(r.block_table)) for r in batch]
        pad = bucket(len(seqs)) - len(seqs)
        steps.append(TraceStep(len(steps), "decode", Batch(seqs, pad, stream=len(steps)), preempted, False,
                               [r.rid for r in batch], [r.length for r in batch]))
        for r in batch:
            r.num_cached = r.length
            r.generated += 1
        finished = [r for r in running if r.generated >= r.output_len]
        for r in finished:
            r.done = True
            pool.release(r.block_table)
            r.block_table = []
        running = [r for r in running if not r.done]
    return steps, reqs, pool
