"""Runs a synthetic workload on the GPU through the C ABI.

Used by the GPU tests, ``bench.py`` and the smoke check. It only moves data
and calls ``binding``: step metadata comes from the library's own
``pkv_prepare_step`` and every device computation from its kernels. Random
values come from the shared seeded generator in ``workloads``.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

import workloads as W

from . import binding as B

NAN_BF16 = 0x7FC0  # quiet NaN bit pattern used to poison unwritten cache rows

_HIP = None
_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


def _hip():
    global _HIP
    if _HIP is None:
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = lib
    return _HIP


class TimingEvent:
    """A HIP event for timing, created with hipEventDisableSystemFence: recording it neither writes back nor
    invalidates the GPU caches. (torch's events carry a system-scope fence; on MI355X two of them around each
    decode call added about 3 us of GPU time per step and slowed the call itself by about 1.5 us.) The event
    still completes only after the work recorded before it, so it can also guard the reuse of a pinned host
    buffer that this work read. Same methods as torch.cuda.Event: record() on the current stream,
    synchronize(), elapsed_time(end) in milliseconds."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        st = _hip().hipEventCreateWithFlags(ctypes.byref(self._h), _EVENT_DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        st = _hip().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def synchronize(self):
        st = _hip().hipEventSynchronize(self._h)
        if st != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({st})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        st = _hip().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if _HIP is not None and self._h:
            _HIP.hipEventDestroy(self._h)


def poisoned_cache(w: W.Workload, device="cuda") -> torch.Tensor:
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    t.view(torch.int16).fill_(NAN_BF16)
    return t


def meta(w: W.Workload, batch: W.Batch, out=None) -> B.StepMeta:
    return B.pkv_prepare_step([s.seq_len for s in batch.seqs], [s.num_cached for s in batch.seqs],
                              [s.block_table for s in batch.seqs], w.block_size, w.max_blocks_per_seq,
                              batch.num_pad, out=out)


class DeviceMeta:
    """Device copies of one batch's metadata; with ``heads`` = (H_q, H_kv)
    also the prefill work plan built from it on the host."""

    def __init__(self, m: B.StepMeta, device="cuda", heads=None):
        self.host = m
        self.slot_mapping = torch.from_numpy(np.ascontiguousarray(m.slot_mapping)).to(device)
        self.cu_seqlens_q = torch.from_numpy(np.ascontiguousarray(m.cu_seqlens_q)).to(device)
        self.context_lens = torch.from_numpy(np.ascontiguousarray(m.context_lens)).to(device)
        self.block_tables = torch.from_numpy(np.ascontiguousarray(m.block_tables)).to(device)
        self.max_q_len = m.max_q_len
        self.max_context_len = m.max_context_len
        self.num_tokens = m.num_tokens
        self.work_items = None
        if heads is not None:
            plan = B.pkv_prefill_plan(m.cu_seqlens_q, m.context_lens, heads[0], heads[1])
            self.work_items = torch.from_numpy(np.ascontiguousarray(plan)).to(device)


class DeviceWorkload:
    """Poisoned caches, setup stores, the step's store and attention passes."""

    def __init__(self, w: W.Workload, device="cuda"):
        self.w = w
        self.device = device
        self.k_cache = poisoned_cache(w, device)
        self.v_cache = poisoned_cache(w, device)

    # -- stores --------------------------------------------------------------
    def run_setup(self):
        for b in self.w.setup:
            k, v = W.batch_kv(self.w, b, self.device)
            m = DeviceMeta(meta(self.w, b), self.device)
            B.kv_store(k, v, self.k_cache, self.v_cache, m.slot_mapping)

    def store_slots(self) -> torch.Tensor:
        slots = meta(self.w, self.w.store).slot_mapping
        mask = W.real_row_mask(self.w)
        full = np.full(mask.size, -1, dtype=np.int32)
        full[mask] = slots
        return torch.from_numpy(full).to(self.device)

    def run_store(self):
        k, v = W.store_kv(self.w, self.device)
        B.kv_store(k, v, self.k_cache, self.v_cache, self.store_slots())

    def build(self):
        self.run_setup()
        self.run_store()
        return self

    # -- attention -----------------------------------------------------------
    def pass_inputs(self, p: W.Pass):
        q = W.pass_q(self.w, p, self.device)
        heads = (self.w.num_q_heads, self.w.num_kv_heads) if p.kind == "prefill" else None
        return q, DeviceMeta(meta(self.w, p.batch), self.device, heads)

    def run_pass(self, p: W.Pass, q=None, m: DeviceMeta = None, out=None, workspace=None, plan=True):
        """plan=False runs prefill on the full grid instead of the host plan."""
        if q is None or m is None:
            q, m = self.pass_inputs(p)
        if out is None:
            out = torch.empty_like(q)
        if p.kind == "decode":
            if workspace is None:
                workspace = decode_workspace(self.w, q.shape[0], m.max_context_len, self.device)
            B.paged_attn_decode(out, q, self.k_cache, self.v_cache, m.block_tables, m.context_lens, self.w.scale,
                                m.max_context_len, workspace)
        else:
            B.paged_attn_prefill_varlen(out, q, m.cu_seqlens_q, m.context_lens, self.k_cache, self.v_cache,
                                        m.block_tables, m.max_q_len, m.max_context_len, self.w.scale,
                                        work_items=m.work_items if plan else None)
        return out


def decode_workspace(w: W.Workload, num_seqs: int, max_ctx: int, device="cuda") -> torch.Tensor:
    n = B.paged_attn_decode_workspace_size(num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, max_ctx)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


class StepRunner:
    """One engine step of a single-pass workload, as an engine runs it:
    host step preparation into pinned buffers, asynchronous upload of the
    metadata, the store of the step's K/V, then the attention pass.

    Two pinned buffer sets alternate, so the host may prepare step i + 1
    while step i is still on the GPU; an event guards each set's reuse."""

    def __init__(self, dw: DeviceWorkload, p: W.Pass):
        self.dw, self.p, w = dw, p, dw.w
        dev = dw.device
        self.q = W.pass_q(w, p, dev)
        self.k, self.v = W.store_kv(w, dev)
        self.out = torch.empty_like(self.q)
        m0 = meta(w, p.batch)
        rows = len(p.batch.seqs) + p.batch.num_pad
        # one int32 buffer holds slot mapping | cu_seqlens_q | context lens |
        # block tables | prefill plan, so a step uploads its metadata with a
        # single copy (the plan starts at an even offset: 8-byte items)
        cap = B.prefill_plan_capacity(m0.num_tokens, rows, w.num_q_heads, w.num_kv_heads)
        head = m0.num_tokens + 2 * rows + 1 + rows * w.max_blocks_per_seq
        self.shapes = (m0.num_tokens, rows + 1, rows, rows * w.max_blocks_per_seq, head & 1,
                       2 * cap if p.kind == "prefill" else 0)
        offs = np.concatenate([[0], np.cumsum(self.shapes)]).astype(np.int64)
        self.offs = offs
        total = int(offs[-1])
        self.pinned = [torch.empty(total, dtype=torch.int32).pin_memory() for _ in range(2)]
        self.events = [None, None]
        self.dev_flat = torch.empty(total, dtype=torch.int32, device=dev)
        self.dev_meta = tuple(self.dev_flat[offs[i]:offs[i + 1]] for i in range(4))
        self.dev_plan = self.dev_flat[offs[5]:offs[6]]
        self.num_items = 0
        self.max_q_len = m0.max_q_len
        self.max_ctx = m0.max_context_len
        self.workspace = (decode_workspace(w, rows, self.max_ctx, dev) if p.kind == "decode" else None)
        # the batch's sequence state as arrays (as a scheduler holds it), one preparation per pinned buffer set
        b = p.batch
        heads = (w.num_q_heads, w.num_kv_heads) if p.kind == "prefill" else None
        self.preps = []
        for k in range(2):
            flat = self.pinned[k].numpy()
            self.preps.append(B.StepPrep([s.seq_len for s in b.seqs], [s.num_cached for s in b.seqs],
                                         [s.block_table for s in b.seqs], w.block_size, w.max_blocks_per_seq,
                                         b.num_pad, tuple(flat[offs[i]:offs[i + 1]] for i in range(4)), heads,
                                         flat[offs[5]:offs[6]]))
        self.i = 0

    def prepare_and_upload(self, record_guard: bool = True) -> int:
        """Host step preparation (pkv_prepare_step, plus pkv_prefill_plan for a
        prefill step) into the next pinned buffer set, then one upload.
        Returns the buffer set used. With record_guard=False the caller
        records, after this step's work, the event that guards the set's
        reuse (``guard(k, event)``), so the step enqueues no extra marker."""
        k = self.i & 1
        self.i += 1
        if self.events[k] is not None:
            self.events[k].synchronize()
        _, self.num_items = self.preps[k]()
        self.dev_flat.copy_(self.pinned[k], non_blocking=True)
        self.events[k] = None
        if record_guard:
            ev = torch.cuda.Event()
            ev.record()
            self.events[k] = ev
        return k

    def guard(self, k: int, event):
        """An event recorded after buffer set k's upload guards its reuse."""
        self.events[k] = event

    def store_only(self):
        slots = self.dev_meta[0]
        B.kv_store(self.k, self.v, self.dw.k_cache, self.dw.v_cache, slots)

    def attention_only(self):
        w = self.dw.w
        _, cu, ctx, bt = self.dev_meta
        bt2 = bt.view(-1, w.max_blocks_per_seq)
        if self.p.kind == "decode":
            B.paged_attn_decode(self.out, self.q, self.dw.k_cache, self.dw.v_cache, bt2, ctx, w.scale,
                                self.max_ctx, self.workspace)
        else:
            items = self.dev_plan[:2 * self.num_items].view(self.num_items, 2)
            B.paged_attn_prefill_varlen(self.out, self.q, cu, ctx, self.dw.k_cache, self.dw.v_cache, bt2,
                                        self.max_q_len, self.max_ctx, w.scale, work_items=items)

    def fused_only(self):
        """The store and the attention in one call (paged_attn_decode_store, paged_attn_prefill_store)."""
        w = self.dw.w
        slots, cu, ctx, bt = self.dev_meta
        bt2 = bt.view(-1, w.max_blocks_per_seq)
        if self.p.kind == "decode":
            B.paged_attn_decode_store(self.out, self.q, self.k, self.v, slots, self.dw.k_cache, self.dw.v_cache, bt2,
                                      ctx, w.scale, self.max_ctx, self.workspace)
        else:
            items = self.dev_plan[:2 * self.num_items].view(self.num_items, 2)
            B.paged_attn_prefill_store(self.out, self.q, self.k, self.v, slots, self.dw.k_cache, self.dw.v_cache, cu,
                                       ctx, bt2, self.max_q_len, self.max_ctx, w.scale, work_items=items)

    def kernels(self):
        self.store_only()
        self.attention_only()

    def step(self):
        self.prepare_and_upload()
        self.kernels()


class TraceRunner:
    """Replays the steps of the native scheduler (``binding.Scheduler``) over
    several layers: each step prepares its metadata on the host once, then
    for every layer draws fresh seeded q/k/v, stores the step's K/V into that
    layer's caches and runs prefill or decode attention."""

    def __init__(self, seed: int, num_layers: int, num_blocks: int, max_blocks_per_seq: int = 8,
                 num_q_heads: int = 16, num_kv_heads: int = 8, head_dim: int = 128, device="cuda"):
        self.seed, self.L, self.device = seed, num_layers, device
        self.hq, self.hkv, self.d, self.mb = num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq
        self.shape_w = W.Workload("trace", seed, num_q_heads, num_kv_heads, head_dim, W.BLOCK_SIZE, num_blocks,
                                  max_blocks_per_seq, [], W.Batch([]), [])
        self.caches = [(poisoned_cache(self.shape_w, device), poisoned_cache(self.shape_w, device))
                       for _ in range(num_layers)]
        ws = B.paged_attn_decode_workspace_size(512, num_q_heads, num_kv_heads, head_dim,
                                                max_blocks_per_seq * W.BLOCK_SIZE)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        self.scale = self.shape_w.scale

    def values(self, step_index: int, layer: int, rows: int):
        from workloads.sched import step_stream
        s = step_stream(step_index, layer)
        q = W.randn_bf16(self.seed, s, W.TAG_Q, (rows, self.hq, self.d), self.device)
        k = W.randn_bf16(self.seed, s, W.TAG_K, (rows, self.hkv, self.d), self.device)
        v = W.randn_bf16(self.seed, s, W.TAG_V, (rows, self.hkv, self.d), self.device)
        return q, k, v

    def run(self, steps, keep=None, timing=None, fused=False):
        """steps: ``binding.SchedStep`` list (step i has index i). keep:
        {step index: layers} whose attention outputs are returned (on the
        host) as {(step index, layer): tensor}. timing: a list that receives
        (step index, layer, e0, e1, e2): HIP events recorded on the current
        stream before the layer's store, between store and attention, and
        after attention (the q/k/v draws stay outside). fused: every
        step stores inside its attention call (paged_attn_decode_store,
        paged_attn_prefill_store; e0 and e1 then mark the same point)."""
        kept = {}
        for i, st in enumerate(steps):
            m = B.pkv_prepare_step(st.seq_lens, st.num_cached, st.block_tables, W.BLOCK_SIZE, self.mb, st.num_pad)
            dm = DeviceMeta(m, self.device, (self.hq, self.hkv) if st.kind == "prefill" else None)
            for layer in range(self.L):
                q, k, v = self.values(i, layer, m.num_tokens)
                kc, vc = self.caches[layer]
                if timing is not None:
                    ev = [TimingEvent() for _ in range(3)]
                    ev[0].record()
                if not fused:
                    B.kv_store(k, v, kc, vc, dm.slot_mapping)
                if timing is not None:
                    ev[1].record()
                out = torch.empty_like(q)
                if fused and st.kind == "decode":
                    B.paged_attn_decode_store(out, q, k, v, dm.slot_mapping, kc, vc, dm.block_tables, dm.context_lens,
                                              self.scale, dm.max_context_len, self.workspace)
                elif fused:
                    B.paged_attn_prefill_store(out, q, k, v, dm.slot_mapping, kc, vc, dm.cu_seqlens_q, dm.context_lens,
                                               dm.block_tables, dm.max_q_len, dm.max_context_len, self.scale,
                                               work_items=dm.work_items)
                elif st.kind == "decode":
                    B.paged_attn_decode(out, q, kc, vc, dm.block_tables, dm.context_lens, self.scale,
                                        dm.max_context_len, self.workspace)
                else:
                    B.paged_attn_prefill_varlen(out, q, dm.cu_seqlens_q, dm.context_lens, kc, vc,
                                                dm.block_tables, dm.max_q_len, dm.max_context_len, self.scale,
                                                work_items=dm.work_items)
                if timing is not None:
                    ev[2].record()
                    timing.append((i, layer, ev[0], ev[1], ev[2]))
                if keep and layer in keep.get(i, ()):
                    kept[(i, layer)] = out.cpu()
        return kept
