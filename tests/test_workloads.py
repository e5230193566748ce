"""Seeded workload generators: reproducibility, shapes and the structural
properties the configurations promise (no GPU)."""

from __future__ import annotations

import numpy as np
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
