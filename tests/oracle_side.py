"""Runs a synthetic workload through the fp64 oracle (host side of parity tests).

Every array the oracle sees is built here from the seeded generator in
``workloads`` with the oracle's own step preparation and store; nothing comes
from the HIP path.
"""

from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import paged as op

NAN_BF16 = np.uint16(0x7FC0)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def metadata(w: W.Workload, batch: W.Batch):
    return op.prepare_step_ref([s.seq_len for s in batch.seqs],
                               [s.num_cached for s in batch.seqs],
                               [s.block_table for s in batch.seqs],
                               w.block_size, w.max_blocks_per_seq, batch.num_pad)


def store_slots(w: W.Workload) -> np.ndarray:
    slots = metadata(w, w.store)[0]
    mask = W.real_row_mask(w)
    out = np.full(mask.size, -1, dtype=np.int32)
    out[mask] = slots
    return out


def empty_caches(w: W.Workload):
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    return np.full(shape, NAN_BF16, dtype=np.uint16), np.full(shape, NAN_BF16, dtype=np.uint16)


def build_caches(w: W.Workload, device="cpu"):
    """Poisoned caches after the setup stores and the step's store."""
    kc, vc = empty_caches(w)
    if w.setup:
        # setup batches write disjoint slots (the oracle's store rejects
        # duplicates), so they are applied as one store
        ks, vs, ss = [], [], []
        for b in w.setup:
            k, v = W.batch_kv(w, b, device)
            ks.append(bits(k)); vs.append(bits(v)); ss.append(metadata(w, b)[0])
        kc, vc = op.kv_store_ref(kc, vc, np.concatenate(ks), np.concatenate(vs), np.concatenate(ss))
    k, v = W.store_kv(w, device)
    kc, vc = op.kv_store_ref(kc, vc, bits(k), bits(v), store_slots(w))
    return kc, vc


def run_pass(w: W.Workload, p: W.Pass, kc, vc, device="cpu", q=None) -> np.ndarray:
    if q is None:
        q = W.pass_q(w, p, device)
    _, cu, ctx, bt = metadata(w, p.batch)
    if p.kind == "decode":
        return op.decode_ref(bits(q), kc, vc, bt, ctx, w.scale)
    return op.prefill_ref(bits(q), cu, ctx, kc, vc, bt, w.scale)


def decode_sampled(w: W.Workload, idx, device="cpu") -> np.ndarray:
    """Oracle decode outputs for the sequences ``idx`` of a decode workload
    whose setup holds one history batch per sequence (configs 2 and 4).

    The chosen sequences' blocks are relabelled into a compact pool (outputs
    do not depend on physical block ids, a pinned oracle property), their
    history and new-token rows are regenerated from the seeded generator and
    stored with the oracle's own store."""
    p = w.passes[0]
    step = p.batch
    q_all = W.pass_q(w, p, device)
    k_new, v_new = W.store_kv(w, device)
    relabel = {}
    tables = []
    for b in idx:
        t = []
        for blk in step.seqs[b].block_table:
            relabel.setdefault(blk, len(relabel))
            t.append(relabel[blk])
        tables.append(t)
    shape = (len(relabel), w.block_size, w.num_kv_heads, w.head_dim)
    kc = np.full(shape, NAN_BF16, dtype=np.uint16)
    vc = np.full(shape, NAN_BF16, dtype=np.uint16)
    seqs_hist, seqs_new = [], []
    hist_k, hist_v, new_k, new_v = [], [], [], []
    for j, b in enumerate(idx):
        s = step.seqs[b]
        hb = w.setup[b]
        k, v = W.batch_kv(w, hb, device)
        hist_k.append(bits(k)); hist_v.append(bits(v))
        seqs_hist.append((s.num_cached, 0, tables[j]))
        seqs_new.append((s.seq_len, s.num_cached, tables[j]))
        new_k.append(bits(k_new[b:b + 1])); new_v.append(bits(v_new[b:b + 1]))
    mb = max(len(t) for t in tables)
    for seqs, ks, vs in ((seqs_hist, hist_k, hist_v), (seqs_new, new_k, new_v)):
        slots, _, _, _ = op.prepare_step_ref([a for a, _, _ in seqs], [c for _, c, _ in seqs],
                                             [t for _, _, t in seqs], w.block_size, mb)
        kc, vc = op.kv_store_ref(kc, vc, np.concatenate(ks), np.concatenate(vs), slots)
    bt = np.full((len(idx), mb), -1, dtype=np.int32)
    for j, t in enumerate(tables):
        bt[j, :len(t)] = t
    ctx = np.asarray([step.seqs[b].seq_len for b in idx], dtype=np.int32)
    q = bits(q_all[list(idx)])
    return op.decode_ref(q, kc, vc, bt, ctx, w.scale)


def trace_check(runner, steps, kept, layers, device="cuda"):
    """Mirror ``layers`` of a scheduler-trace replay on the host with the
    oracle's own metadata and in-place store, and compare the outputs the GPU
    kept at sampled steps. Returns the number of (step, layer) checks made."""
    from tests.test_gpu_parity import assert_close
    shape = (runner.shape_w.num_blocks, runner.shape_w.block_size, runner.hkv, runner.d)
    mirror = {l: (np.full(shape, NAN_BF16, dtype=np.uint16), np.full(shape, NAN_BF16, dtype=np.uint16))
              for l in layers}
    checked = 0
    for st in steps:
        b = st.batch
        slots, cu, ctx, bt = op.prepare_step_ref([s.seq_len for s in b.seqs], [s.num_cached for s in b.seqs],
                                                 [s.block_table for s in b.seqs], runner.shape_w.block_size,
                                                 runner.mb, b.num_pad)
        for l in layers:
            q, k, v = runner.values(st.index, l, len(slots))
            kc, vc = mirror[l]
            op.kv_store_inplace_ref(kc, vc, bits(k), bits(v), slots)
            if (st.index, l) in kept:
                if st.kind == "decode":
                    ref = op.decode_ref(bits(q), kc, vc, bt, ctx, runner.scale)
                else:
                    ref = op.prefill_ref(bits(q), cu, ctx, kc, vc, bt, runner.scale)
                assert_close(kept[(st.index, l)], ref, cu, f"trace step {st.index} ({st.kind}) layer {l}")
                checked += 1
    return checked
