"""Seeded synthetic workloads shared by the oracle side and the HIP side.

This module plays the part of the engine's block manager and scheduler: it
draws sequence lengths, cached-prefix lengths and block tables from a shuffled
block pool, and it draws the random bf16 values. It holds none of the method's
arithmetic: it computes no slot, no metadata array handed to a kernel, and no
attention. Each side turns a ``Workload`` into kernel inputs with its own
code (the oracle with ``oracle.prepare_step_ref``, the HIP side with the
library's own step preparation).

Page references: P1 = "13. 读一个最小推理引擎：nano-vllm".

Workloads (shapes follow a Qwen3-0.6B-like attention layer):
  1 tiny      4 sequences (37/256/300/511), one store with interleaved -1 rows,
              one decode pass and one prefill pass (cached 0/0/256/256).
  2 decode    256 sequences, context U[100, 2048], padded to 272 rows.
  3 prefill   16384-token budget of varlen prompts U[100, 1024]; about half
              carry a 256/512-token prefix in shared refcounted blocks; the
              first is a chunk continuation cut mid-block.
  4 long      512 sequences, context U[4096, 32768], 32 Q / 8 KV heads.
  5 trace     request lengths for the FCFS prefill-first replay over 28 layers (``workloads.sched``).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 256
HEAD_DIM = 128
SEEDS = {1: 0, 2: 1, 3: 2, 4: 3, 5: 4}


@dataclass
class Seq:
    """One sequence's state at a step: the step computes tokens
    [num_cached, seq_len) and the context it attends to is [0, seq_len)
    (P1, "第二站：一个请求的状态")."""
    seq_len: int
    num_cached: int
    block_table: list


@dataclass
class Batch:
    """A group of sequences whose new tokens are stored (and attended) together.

    ``stream`` selects the random stream of this batch's K/V rows (and of its
    queries for an attention pass). ``num_pad`` padding rows follow the real
    sequences (decode batch padded up to a replay bucket, P1 "第五站")."""
    seqs: list
    num_pad: int = 0
    stream: int = 0

    @property
    def num_rows(self) -> int:
        return sum(s.seq_len - s.num_cached for s in self.seqs) + self.num_pad


@dataclass
class Pass:
    """An attention pass run after the step's store."""
    kind: str            # "decode" or "prefill"
    batch: Batch


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    setup: list                      # Batches stored before the step (history, shared prefixes)
    store: Batch                     # the step's store
    passes: list                     # Passes run after the store
    pad_positions: list = field(default_factory=list)  # store rows that are -1 rows interleaved
    shared_blocks: dict = field(default_factory=dict)  # physical block -> refcount (read-only)
    # value shaping for softmax edge cases (defaults leave the N(0, 1) draws as they are):
    # q = q_mult * z + q_bias and K at position p = z + k_ramp * p, in fp32 before the bf16 rounding
    q_mult: float = 1.0
    q_bias: float = 0.0
    k_ramp: float = 0.0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D). The pages do not state it; this is the
        usual attention scale."""
        return 1.0 / float(np.sqrt(self.head_dim))

    def store_rows(self) -> int:
        return self.store.num_rows + len(self.pad_positions)


# ----------------------------------------------------------------------------
# random values
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def randn_f32(seed: int, stream: int, tag: int, shape, device="cpu"):
    """fp32 N(0, 1) draws from a generator seeded by (seed, stream, tag). The
    same call on the same device returns the same tensor; CPU and GPU
    generators produce different streams."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 40) ^ (int(stream) << 4) ^ int(tag))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)


def randn_bf16(seed: int, stream: int, tag: int, shape, device="cpu"):
    """``randn_f32`` rounded to bf16 (nearest even)."""
    return randn_f32(seed, stream, tag, shape, device).to(_torch().bfloat16)


TAG_K, TAG_V, TAG_Q = 1, 2, 3


def row_positions(batch: Batch, extra_rows: int = 0) -> np.ndarray:
    """Context position of every row of a batch's K/V block (the sequences'
    tokens num_cached .. seq_len - 1 in order, then 0 for padding rows)."""
    parts = [np.arange(s.num_cached, s.seq_len) for s in batch.seqs]
    parts.append(np.zeros(batch.num_pad + extra_rows, dtype=np.int64))
    return np.concatenate(parts).astype(np.float32)


def batch_kv(w: Workload, batch: Batch, device="cpu", extra_rows: int = 0):
    """K and V rows for a batch: [rows, H_kv, D] bf16 each (K shaped by
    ``w.k_ramp`` when set)."""
    torch = _torch()
    rows = batch.num_rows + extra_rows
    shape = (rows, w.num_kv_heads, w.head_dim)
    v = randn_bf16(w.seed, batch.stream, TAG_V, shape, device)
    if not w.k_ramp:
        return randn_bf16(w.seed, batch.stream, TAG_K, shape, device), v
    if w.pad_positions:
        raise ValueError("k_ramp needs padding rows at the end of the batch")
    k = randn_f32(w.seed, batch.stream, TAG_K, shape, device)
    pos = torch.from_numpy(row_positions(batch, extra_rows)).to(device)
    return (k + w.k_ramp * pos[:, None, None]).to(torch.bfloat16), v


def pass_q(w: Workload, p: Pass, device="cpu"):
    """Query rows for an attention pass: [rows, H_q, D] bf16 (scaled and
    shifted by ``w.q_mult`` / ``w.q_bias`` when set)."""
    shape = (p.batch.num_rows, w.num_q_heads, w.head_dim)
    if w.q_mult == 1.0 and w.q_bias == 0.0:
        return randn_bf16(w.seed, p.batch.stream + 500_000, TAG_Q, shape, device)
    q = randn_f32(w.seed, p.batch.stream + 500_000, TAG_Q, shape, device)
    return (q * w.q_mult + w.q_bias).to(_torch().bfloat16)


def store_kv(w: Workload, device="cpu"):
    """K/V rows of the step's store, including interleaved padding rows."""
    return batch_kv(w, w.store, device, extra_rows=len(w.pad_positions))


# ----------------------------------------------------------------------------
# block pool
# ----------------------------------------------------------------------------

class _Pool:
    """Physical blocks handed out in the order of a seeded permutation."""

    def __init__(self, rng, num_blocks: int):
        self.order = [int(x) for x in rng.permutation(num_blocks)]
        self.next = 0

    def take(self, n: int) -> list:
        if self.next + n > len(self.order):
            raise RuntimeError("pool exhausted")
        out = self.order[self.next:self.next + n]
        self.next += n
        return out


def _blocks_for(L: int, bs: int = BLOCK_SIZE) -> int:
    return -(-L // bs)


# ----------------------------------------------------------------------------
# the five configurations
# ----------------------------------------------------------------------------

def tiny(seed: int = SEEDS[1]) -> Workload:
    """Config 1: 4 sequences, 16-block pool, one store of every context token
    with 16 padding rows interleaved, then a decode and a prefill pass."""
    rng = np.random.default_rng(seed)
    lens = [37, 256, 300, 511]
    cached_prefill = [0, 0, 256, 256]
    pool = _Pool(rng, 16)
    tables = [pool.take(_blocks_for(L)) for L in lens]
    store = Batch([Seq(L, 0, t) for L, t in zip(lens, tables)], stream=1)
    total = store.num_rows + 16
    pad_positions = sorted(int(x) for x in rng.choice(total, size=16, replace=False))
    decode = Pass("decode", Batch([Seq(L, L - 1, t) for L, t in zip(lens, tables)], stream=2))
    prefill = Pass("prefill", Batch([Seq(L, c, t) for L, c, t in zip(lens, cached_prefill, tables)],
                                    stream=3))
    return Workload("tiny", seed, 16, 8, HEAD_DIM, BLOCK_SIZE, 16, 2, [], store,
                    [decode, prefill], pad_positions)


def _decode_workload(name, seed, batch, lo, hi, hq, num_pad, pool_factor=1.25) -> Workload:
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(lo, hi + 1, size=batch)]
    need = sum(_blocks_for(L) for L in lens)
    num_blocks = int(np.ceil(pool_factor * need))
    pool = _Pool(rng, num_blocks)
    tables = [pool.take(_blocks_for(L)) for L in lens]
    setup = [Batch([Seq(L - 1, 0, t)], stream=10 + i) for i, (L, t) in enumerate(zip(lens, tables))]
    step = Batch([Seq(L, L - 1, t) for L, t in zip(lens, tables)], num_pad=num_pad, stream=1)
    mb = _blocks_for(hi)
    return Workload(name, seed, hq, 8, HEAD_DIM, BLOCK_SIZE, num_blocks, mb, setup, step,
                    [Pass("decode", step)])


def decode(seed: int = SEEDS[2]) -> Workload:
    """Config 2: 256 sequences, context U[100, 2048], 16 Q / 8 KV heads, pool
    1.25x the blocks needed, batch padded to 272 rows with -1 slots."""
    return _decode_workload("decode", seed, 256, 100, 2048, 16, 16)


def long_decode(seed: int = SEEDS[4]) -> Workload:
    """Config 4: 512 sequences, context U[4096, 32768], 32 Q / 8 KV heads."""
    return _decode_workload("long_decode", seed, 512, 4096, 32768, 32, 0)


def chunked_prefill(seed: int = SEEDS[3], budget: int = 16384) -> Workload:
    """Config 3: prompts U[100, 1024] added while the new-token budget allows.

    * Four shared prefix groups (two of one block, two of two blocks) are
      written once at setup and referenced, read-only, by the sequences that
      carry a prefix (refcount = number of such sequences).
    * A sequence other than the first carries a prefix with probability 1/2
      when its length exceeds 256 tokens: 512 tokens (only if longer than
      512, probability 1/2) or else 256.
    * The first sequence continues a chunked prefill: its first c0 tokens
      (1 <= c0 < L0, c0 not a multiple of 256) are in its own blocks.
    """
    rng = np.random.default_rng(seed)
    bs = BLOCK_SIZE
    # first pass: draw the sequence plan
    plan = []          # (L, cached, group or None)
    total = 0
    L0 = int(rng.integers(100, 1025))
    while True:
        c0 = int(rng.integers(1, L0))
        if c0 % bs:
            break
    plan.append((L0, c0, None))
    total += L0 - c0
    group_len = [256, 256, 512, 512]
    while True:
        L = int(rng.integers(100, 1025))
        grp = None
        if L > 256 and rng.random() < 0.5:
            if L > 512 and rng.random() < 0.5:
                grp = 2 + int(rng.integers(0, 2))
            else:
                grp = int(rng.integers(0, 2))
        c = group_len[grp] if grp is not None else 0
        if total + (L - c) > budget:
            break
        plan.append((L, c, grp))
        total += L - c
    need = 6 + sum(_blocks_for(L) - (c // bs if g is not None else 0) for L, c, g in plan)
    num_blocks = int(np.ceil(1.25 * need))
    pool = _Pool(rng, num_blocks)
    groups = [pool.take(gl // bs) for gl in group_len]
    seqs = []
    setup = [Batch([Seq(gl, 0, groups[i]) for i, gl in enumerate(group_len)], stream=10)]
    shared = {}
    for i, (L, c, g) in enumerate(plan):
        if g is None:
            table = pool.take(_blocks_for(L))
        else:
            table = list(groups[g]) + pool.take(_blocks_for(L) - c // bs)
            for blk in groups[g]:
                shared[blk] = shared.get(blk, 0) + 1
        seqs.append(Seq(L, c, table))
        if i == 0:
            setup.append(Batch([Seq(c, 0, table)], stream=11))
    step = Batch(seqs, stream=1)
    return Workload("chunked_prefill", seed, 16, 8, HEAD_DIM, bs, num_blocks, _blocks_for(1024),
                    setup, step, [Pass("prefill", step)], shared_blocks=shared)


def make(k: int, seed=None) -> Workload:
    """Workload for configuration k (1..4); config 5 lives in ``workloads.sched``."""
    fns = {1: tiny, 2: decode, 3: chunked_prefill, 4: long_decode}
    if k not in fns:
        raise ValueError(f"unknown configuration {k}")
    return fns[k](SEEDS[k] if seed is None else seed)


def real_row_mask(w: Workload) -> np.ndarray:
    """Boolean mask over the step store's rows: False where a padding row
    (slot -1) is interleaved, True for the store batch's rows in order."""
    total = w.store_rows()
    mask = np.ones(total, dtype=bool)
    if w.pad_positions:
        mask[np.asarray(w.pad_positions, dtype=np.int64)] = False
    return mask
