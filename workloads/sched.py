"""Configuration 5: a deterministic FCFS, prefill-first scheduler replay.

Token-free stand-in for the engine loop the pages describe; it decides, step
by step, which sequences run and which blocks they own, and records each
step's sequence states. It computes no slot and no attention (each side
prepares its own step metadata from the recorded states).

Page references, P1 = "13. 读一个最小推理引擎：nano-vllm":

* "第三站：调度器": a step first tries prefill, taking waiting requests in FCFS
  order while the running count stays within max_num_seqs, the token budget
  (max_num_batched_tokens) has room and free blocks suffice; only the first
  request of a step may be cut to the remaining budget (its remainder stays
  at the head of the waiting queue); any prefill makes the step
  prefill-only. Otherwise every running sequence advances one token; when
  blocks run out the most recently added running sequence is preempted: it
  frees all its blocks and goes back to the front of the waiting queue, to
  be recomputed (no swap to host).
* "第四站：块管理与前缀缓存": a request scheduled for the first time gets
  blocks for its whole input at once; a decode step needs a new block
  exactly when len(seq) % block_size == 1; freed blocks return to the free
  queue. Prefix caching needs token ids, which these token-free requests do
  not have, so it is off.
* "第五站：执行准备与 KV 容量": decode batches are padded up to a replay
  bucket (1, 2, 4, 8, then multiples of 16 up to 512).
* "第一站：主循环": a prefill that completes a prompt yields one token; each
  decode step yields one token; a request finishes after output_len tokens.

Readings: a request with output length O therefore runs O - 1 decode steps,
and the K/V of its final token is never stored; a chunked prefill yields no
token until its last chunk; after a preemption the request re-prefills its
prompt plus the tokens generated so far from position 0.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from . import BLOCK_SIZE, Batch, Seq, SEEDS

MAX_NUM_SEQS = 512
MAX_BATCHED_TOKENS = 16384
NUM_LAYERS = 28
POOL_BLOCKS = 800  # per layer; small enough that the replay preempts (23 times at seed 4)
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


def _bucket(n: int) -> int:
    for b in BUCKETS:
        if b >= n:
            return b
    return n


def replay(seed: int = SEEDS[5], num_requests: int = 256, num_blocks: int = POOL_BLOCKS,
           max_num_seqs: int = MAX_NUM_SEQS, budget: int = MAX_BATCHED_TOKENS,
           block_size: int = BLOCK_SIZE, lo: int = 100, hi: int = 1024):
    """Run the schedule to completion; returns (steps, requests, pool)."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(lo, hi + 1, size=num_requests)
    outputs = rng.integers(lo, hi + 1, size=num_requests)
    reqs = [Request(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]
    waiting = deque(reqs)
    running: list = []   # in the order sequences were added
    pool = BlockPool(num_blocks)
    steps = []
    need = lambda L: -(-L // block_size)  # noqa: E731

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
            steps.append(TraceStep(len(steps), "prefill", Batch(seqs, 0, stream=len(steps)), [], chunked,
                                   [r.rid for r, _ in scheduled], [r.length for r, _ in scheduled]))
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
        # ---- decode phase ----
        preempted, batch = [], []
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
            continue
        seqs = [Seq(r.length, r.length - 1, list(r.block_table)) for r in batch]
        pad = _bucket(len(seqs)) - len(seqs)
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


def step_stream(step: int, layer: int) -> int:
    """Random-stream id of a (step, layer) pair's q/k/v."""
    return 1_000_000 + step * 64 + layer
