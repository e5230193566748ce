"""Configuration 5 scheduler replay: the rules the pages state hold on the
recorded trace (no GPU)."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import paged as op
from workloads import sched as S


@pytest.fixture(scope="module")
def trace():
    return S.replay()


def _need(L):
    return -(-L // 256)


def test_deterministic(trace):
    steps2, _, _ = S.replay()
    steps, _, _ = trace
    assert len(steps) == len(steps2)
    for a, b in zip(steps, steps2):
        assert a.kind == b.kind and a.rids == b.rids
        assert [(s.seq_len, s.num_cached, s.block_table) for s in a.batch.seqs] == \
               [(s.seq_len, s.num_cached, s.block_table) for s in b.batch.seqs]


def test_every_request_completes(trace):
    steps, reqs, pool = trace
    assert all(r.done and r.generated == r.output_len for r in reqs)
    assert len(pool.free) == pool.num_blocks and len(set(pool.free)) == pool.num_blocks


def test_budget_batch_and_buckets(trace):
    steps, _, _ = trace
    for st in steps:
        n = sum(s.seq_len - s.num_cached for s in st.batch.seqs)
        if st.kind == "prefill":
            assert n <= S.MAX_BATCHED_TOKENS and st.batch.num_pad == 0
        else:
            assert n == len(st.batch.seqs) <= S.MAX_NUM_SEQS
            total = len(st.batch.seqs) + st.batch.num_pad
            assert total == min(t for t in S.BUCKETS if t >= len(st.batch.seqs))  # smallest bucket that fits


def test_only_first_prefill_may_be_chunked(trace):
    steps, _, _ = trace
    for st in steps:
        if st.kind == "prefill":
            for s, full in zip(st.batch.seqs[1:], st.full_lens[1:]):
                assert s.seq_len == full
            if not st.chunked_first:
                assert st.batch.seqs[0].seq_len == st.full_lens[0]


def test_blocks_disjoint_and_sufficient(trace):
    steps, _, _ = trace
    for st in steps:
        owned = [b for s in st.batch.seqs for b in s.block_table]
        assert len(owned) == len(set(owned))
        for s in st.batch.seqs:
            assert len(s.block_table) >= _need(s.seq_len)
            if st.kind == "decode":
                assert len(s.block_table) == _need(s.seq_len)  # a block is added exactly when len % 256 == 1
        slots = op.prepare_step_ref([s.seq_len for s in st.batch.seqs], [s.num_cached for s in st.batch.seqs],
                                    [s.block_table for s in st.batch.seqs], 256, 8, st.batch.num_pad)[0]
        live = slots[slots >= 0]
        assert np.unique(live).size == live.size


def test_preemption_recomputes_from_scratch(trace):
    steps, reqs, _ = trace
    pre = [(st.index, rid) for st in steps for rid in st.preempted]
    assert len(pre) >= 1
    for idx, rid in pre:
        nxt = next(st for st in steps[idx:] if rid in st.rids)
        assert nxt.kind == "prefill"
        s = nxt.batch.seqs[nxt.rids.index(rid)]
        assert s.num_cached == 0
    # preemption takes the most recently added running sequences: a preempted
    # request never appears before a survivor that joined the batch later
    for st in steps:
        if st.preempted and st.kind == "decode":
            assert not (set(st.preempted) & set(st.rids))


def test_token_accounting(trace):
    steps, reqs, _ = trace
    done_prefills = {r.rid: 0 for r in reqs}
    decodes = {r.rid: 0 for r in reqs}
    for st in steps:
        for s, full, rid in zip(st.batch.seqs, st.full_lens, st.rids):
            if st.kind == "prefill" and s.seq_len == full:
                done_prefills[rid] += 1
            elif st.kind == "decode":
                decodes[rid] += 1
    for r in reqs:
        assert done_prefills[r.rid] + decodes[r.rid] == r.output_len
