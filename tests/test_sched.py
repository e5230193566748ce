"""Scheduler (configuration 5): the oracle against hand-worked schedules and the
rules the pages state, and the native scheduler against the oracle, step for
step (no GPU)."""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import paged_kv_attention_28_amd as P
from oracle import paged as op
from oracle import sched as OS
from workloads import sched as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sched_tiny.json")


@pytest.fixture(scope="module")
def trace():
    p, o = S.requests()
    return OS.replay(p, o, S.POOL_BLOCKS, S.MAX_NUM_SEQS, S.MAX_BATCHED_TOKENS)


def _need(L):
    return -(-L // 256)


def _oracle_rows(st):
    return {"kind": st.kind,
            "seqs": [[rid, s.seq_len, s.num_cached, list(s.block_table)] for rid, s in zip(st.rids, st.batch.seqs)],
            "num_pad": st.batch.num_pad, "chunked_first": bool(st.chunked_first), "preempted": list(st.preempted)}


def _native_rows(st):
    return {"kind": st.kind,
            "seqs": [[rid, L, c, bt] for rid, L, c, bt in zip(st.request_ids, st.seq_lens, st.num_cached,
                                                              st.block_tables)],
            "num_pad": st.num_pad, "chunked_first": st.chunked_first, "preempted": st.preempted}


# ----------------------------------------------------------------------------
# oracle pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_oracle_matches_hand_worked_schedule(case):
    p = [r[0] for r in case["requests"]]
    o = [r[1] for r in case["requests"]]
    steps, reqs, pool = OS.replay(p, o, case["num_blocks"], case["max_num_seqs"], case["budget"],
                                  case["block_size"])
    assert [_oracle_rows(st) for st in steps] == case["steps"]
    assert sorted(pool.free) == list(range(case["num_blocks"]))


def test_oracle_rejects_a_request_larger_than_the_pool():
    # 8 prompt tokens fill both blocks; the first decode needs a third block,
    # preempts the only sequence, and its recompute can never fit
    with pytest.raises(ValueError):
        OS.replay([8], [3], num_blocks=2, max_num_seqs=4, budget=64, block_size=4)


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
            assert total == min(t for t in OS.BUCKETS if t >= len(st.batch.seqs))  # smallest bucket that fits


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
        nxt = next(st for st in steps[idx + 1:] if rid in st.rids)
        assert nxt.kind == "prefill"
        s = nxt.batch.seqs[nxt.rids.index(rid)]
        assert s.num_cached == 0
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


# ----------------------------------------------------------------------------
# native scheduler against the oracle
# ----------------------------------------------------------------------------

def _native(prompts, outputs, num_blocks, max_num_seqs, budget, block_size=256):
    return P.Scheduler(num_blocks, block_size, max_num_seqs, budget).run(prompts, outputs)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_native_matches_hand_worked_schedule(case):
    p = [r[0] for r in case["requests"]]
    o = [r[1] for r in case["requests"]]
    steps = _native(p, o, case["num_blocks"], case["max_num_seqs"], case["budget"], case["block_size"])
    assert [_native_rows(st) for st in steps] == case["steps"]


def test_native_matches_oracle_on_the_replay(trace):
    steps, _, _ = trace
    p, o = S.requests()
    sch = P.Scheduler(S.POOL_BLOCKS, 256, S.MAX_NUM_SEQS, S.MAX_BATCHED_TOKENS)
    nat = sch.run(p, o)
    assert len(nat) == len(steps)
    for a, b in zip(nat, steps):
        assert _native_rows(a) == _oracle_rows(b), b.index
        assert a.full_lens == b.full_lens
    assert sch.unfinished == 0 and sch.free_blocks == S.POOL_BLOCKS


@pytest.mark.parametrize("seed", range(60))
def test_native_matches_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(2, 12))
    bs = int(rng.choice([4, 8, 16]))
    p = rng.integers(1, 40, size=n)
    o = rng.integers(1, 30, size=n)
    nb = int(max(-(-int(p.max() + o.max()) // bs), rng.integers(2, 12)))
    mns = int(rng.integers(1, 6))
    bud = int(rng.integers(4, 64))
    try:
        ref, _, _ = OS.replay(p, o, nb, mns, bud, bs)
    except ValueError:
        with pytest.raises(P.PkvError):
            _native(p, o, nb, mns, bud, bs)
        return
    nat = _native(p, o, nb, mns, bud, bs)
    assert [_native_rows(st) for st in nat] == [_oracle_rows(st) for st in ref]


def test_native_rejects_a_request_larger_than_the_pool():
    sch = P.Scheduler(2, 4, 4, 64)
    sch.add(8, 3)
    assert sch.schedule().kind == "prefill"
    sch.postprocess()
    with pytest.raises(P.PkvError):
        sch.schedule()


def test_native_validation():
    with pytest.raises(P.PkvError):
        P.Scheduler(10, 0, 4, 64)
    with pytest.raises(P.PkvError):
        P.Scheduler(10, 4, 0, 64)
    sch = P.Scheduler(10, 4, 4, 64)
    with pytest.raises(P.PkvError):
        sch.add(0, 3)
    with pytest.raises(P.PkvError):
        sch.add(3, 0)
    with pytest.raises(P.PkvError):
        sch.postprocess()                # nothing scheduled
    sch.add(3, 2)
    assert sch.schedule() is not None
    with pytest.raises(P.PkvError):
        sch.schedule()                   # previous step not postprocessed
    with pytest.raises(P.PkvError):
        sch.add(3, 2)                    # not between schedule and postprocess
    sch.postprocess()
    assert sch.unfinished == 1
    empty = P.Scheduler(10, 4, 4, 64)
    assert empty.schedule() is None and empty.unfinished == 0
