"""Seeded workload generators: reproducibility, shapes and the structural
properties the configurations promise (no GPU)."""

from __future__ import annotations

import numpy as np
import torch
import pytest

import workloads as W
from oracle import paged as op
from tests.oracle_side import metadata, store_slots


def _all_store_slots(w):
    out = [metadata(w, b)[0] for b in w.setup] + [store_slots(w)]
    return np.concatenate(out)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_reproducible(k):
    a, b = W.make(k), W.make(k)
    assert [s.block_table for s in a.store.seqs] == [s.block_table for s in b.store.seqs]
    assert [s.seq_len for s in a.store.seqs] == [s.seq_len for s in b.store.seqs]
    assert a.num_blocks == b.num_blocks


@pytest.mark.parametrize("k", [1, 2, 3])
def test_slots_distinct_and_in_pool(k):
    w = W.make(k)
    s = _all_store_slots(w)
    live = s[s != -1]
    assert live.min() >= 0 and live.max() < w.num_blocks * w.block_size
    assert np.unique(live).size == live.size


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_tables_cover_contexts(k):
    w = W.make(k)
    for p in w.passes:
        for s in p.batch.seqs:
            assert len(s.block_table) >= -(-s.seq_len // w.block_size)
            assert len(s.block_table) <= w.max_blocks_per_seq
            assert all(0 <= x < w.num_blocks for x in s.block_table)
            assert 0 <= s.num_cached < s.seq_len


def test_tiny_shape():
    w = W.make(1)
    assert [s.seq_len for s in w.store.seqs] == [37, 256, 300, 511]
    assert w.store_rows() == 1120 and len(w.pad_positions) == 16
    assert [s.num_cached for s in w.passes[1].batch.seqs] == [0, 0, 256, 256]
    used = sorted(b for s in w.store.seqs for b in s.block_table)
    assert len(used) == 6 and len(set(used)) == 6


def test_decode_shape():
    w = W.make(2)
    lens = [s.seq_len for s in w.store.seqs]
    assert len(lens) == 256 and w.store.num_pad == 16 and w.store.num_rows == 272
    assert min(lens) >= 100 and max(lens) <= 2048
    need = sum(-(-L // 256) for L in lens)
    assert w.num_blocks == int(np.ceil(1.25 * need))
    blocks = [b for s in w.store.seqs for b in s.block_table]
    assert len(set(blocks)) == len(blocks)


def test_long_decode_shape():
    w = W.make(4)
    lens = [s.seq_len for s in w.store.seqs]
    assert len(lens) == 512 and min(lens) >= 4096 and max(lens) <= 32768
    assert w.num_q_heads == 32 and w.num_kv_heads == 8
    assert w.max_blocks_per_seq == 128


def test_chunked_prefill_structure():
    w = W.make(3)
    seqs = w.store.seqs
    new = sum(s.seq_len - s.num_cached for s in seqs)
    assert new <= 16384
    assert all(100 <= s.seq_len <= 1024 for s in seqs)
    s0 = seqs[0]
    assert 1 <= s0.num_cached < s0.seq_len and s0.num_cached % 256 != 0
    prefixed = [s for s in seqs[1:] if s.num_cached > 0]
    assert all(s.num_cached in (256, 512) for s in prefixed)
    assert 0.25 <= len(prefixed) / len(seqs) <= 0.6
    # shared blocks are read-only: never a store target of the step
    step_blocks = {int(x) // 256 for x in store_slots(w) if x != -1}
    assert not (step_blocks & set(w.shared_blocks))
    # refcounts equal the number of sequences referencing the block
    for blk, rc in w.shared_blocks.items():
        assert rc == sum(blk in s.block_table for s in seqs)
    # own blocks of different sequences are disjoint
    owned = [b for s in seqs for b in s.block_table if b not in w.shared_blocks]
    assert len(owned) == len(set(owned))


def test_values_reproducible():
    w = W.make(1)
    k1, v1 = W.store_kv(w)
    k2, v2 = W.store_kv(w)
    assert k1.shape == (1120, 8, 128)
    assert bool((k1 == k2).all()) and bool((v1 == v2).all())
    assert not bool((k1 == v1).all())
    q = W.pass_q(w, w.passes[1])
    assert q.shape == (592, 16, 128)
    x = q.float()
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02


def test_oracle_on_tiny_config_is_finite():
    """Poisoned (NaN) unused rows never reach the oracle's outputs."""
    from tests.oracle_side import build_caches, run_pass
    w = W.make(1)
    kc, vc = build_caches(w)
    for p in w.passes:
        out = run_pass(w, p, kc, vc)
        assert np.isfinite(out).all()
    # unused blocks still hold the poison
    used = {b for s in w.store.seqs for b in s.block_table}
    for blk in range(w.num_blocks):
        if blk not in used:
            assert (kc[blk] == 0x7FC0).all()


def _shaped(lens, hq=16, **kw):
    rng = np.random.default_rng(3)
    nb = [-(-L // 256) for L in lens]
    pool = W._Pool(rng, sum(nb))
    tables = [pool.take(n) for n in nb]
    setup = [W.Batch([W.Seq(L - 1, 0, t) for L, t in zip(lens, tables)], stream=5)]
    step = W.Batch([W.Seq(L, L - 1, t) for L, t in zip(lens, tables)], stream=6)
    w = W.Workload("shaped", 7, hq, 8, 128, 256, sum(nb), max(nb), setup, step, [W.Pass("decode", step)])
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def test_value_shaping_defaults_leave_draws_unchanged():
    w = _shaped([300, 40])
    k, v = W.batch_kv(w, w.setup[0])
    assert torch.equal(k.view(torch.int16), W.randn_bf16(w.seed, 5, W.TAG_K, k.shape).view(torch.int16))
    q = W.pass_q(w, w.passes[0])
    assert torch.equal(q.view(torch.int16), W.randn_bf16(w.seed, 6 + 500_000, W.TAG_Q, q.shape).view(torch.int16))


def test_ramp_moves_the_running_max_on_every_key_tile():
    """The rising-score workload used by the GPU edge cases does what it is for: for every query head, the
    largest score (log2 units, scale 1/sqrt(128)) of each 32-key tile beats every earlier tile's by more than
    8, so a lazily rescaled running max has to move on every tile."""
    w = _shaped([2000], q_bias=1.0, k_ramp=0.03)
    k, _ = W.batch_kv(w, w.setup[0])
    q = W.pass_q(w, w.passes[0])
    s = np.einsum("hd,lhd->hl", q[0].double().numpy().reshape(8, 2, 128)[:, 0], k.double().numpy())
    s *= w.scale / np.log(2.0)
    tiles = s[:, : 1984].reshape(8, -1, 32).max(axis=2)
    rise = tiles[:, 1:] - np.maximum.accumulate(tiles, axis=1)[:, :-1]
    assert rise.min() > 8.0, rise.min()


def test_peaky_queries_widen_the_scores():
    """q x 8: the scores' spread is about 8 times that of the plain draws (a softmax dominated by few keys)."""
    w1, w8 = _shaped([1500]), _shaped([1500], q_mult=8.0)
    k, _ = W.batch_kv(w1, w1.setup[0])
    spread = []
    for w in (w1, w8):
        q = W.pass_q(w, w.passes[0])
        s = np.einsum("hd,lhd->hl", q[0].double().numpy()[::2], k.double().numpy()) * w.scale
        spread.append(s.std())
    assert 7.5 < spread[1] / spread[0] < 8.5
