"""ctypes binding of libpkv.so: the same names as the C ABI in ``include/pkv.h``.

Argument marshalling only: tensors are checked (dtype, device, contiguity) and
passed as raw pointers together with torch's current HIP stream. Every step of
the path runs in the library. There is no fallback: if libpkv.so is missing
or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_OK = 0
STATUS = {0: "OK", 1: "INVALID", 2: "UNSUPPORTED", 3: "HIP", 4: "WORKSPACE"}

EXPORTS = ("pkv_last_error", "pkv_abi_version", "pkv_prepare_step", "kv_store",
           "paged_attn_decode_workspace_size", "paged_attn_decode", "paged_attn_decode_noalloc",
           "paged_attn_decode_store",
           "paged_attn_prefill_varlen", "paged_attn_prefill_store",
           "pkv_prefill_plan", "pkv_sched_create", "pkv_sched_destroy", "pkv_sched_add", "pkv_sched_schedule",
           "pkv_sched_postprocess", "pkv_sched_unfinished", "pkv_sched_free_blocks", "pkv_decode_graphs_create",
           "pkv_decode_graphs_create_layers",
           "pkv_decode_graphs_launch", "pkv_decode_graphs_destroy", "rope_kv_store", "pkv_rope_cos_sin",
           "sample_temperature_workspace_size", "sample_temperature")
ABI_VERSION = 10


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


class DecodeGraphDesc(ctypes.Structure):
    """pkv_decode_graph_desc (include/pkv.h)."""
    _fields_ = [("key", ctypes.c_void_p), ("key_stride", ctypes.c_int64), ("value", ctypes.c_void_p),
                ("value_stride", ctypes.c_int64), ("slot_mapping", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("num_blocks", ctypes.c_int64), ("q", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("context_lens", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("scale", ctypes.c_float), ("max_context_len", ctypes.c_int32)]


class SchedBatch(ctypes.Structure):
    """pkv_sched_batch (include/pkv.h)."""
    _fields_ = [("kind", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("num_pad", ctypes.c_int32),
                ("chunked_first", ctypes.c_int32), ("num_preempted", ctypes.c_int32),
                ("request_ids", ctypes.POINTER(ctypes.c_int32)), ("seq_lens", ctypes.POINTER(ctypes.c_int32)),
                ("num_cached", ctypes.POINTER(ctypes.c_int32)), ("full_lens", ctypes.POINTER(ctypes.c_int32)),
                ("bt_offsets", ctypes.POINTER(ctypes.c_int64)), ("bt_data", ctypes.POINTER(ctypes.c_int32)),
                ("preempted", ctypes.POINTER(ctypes.c_int32))]

c_i32, c_i64, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
P_I32 = ctypes.POINTER(ctypes.c_int32)
P_I64 = ctypes.POINTER(ctypes.c_int64)


def load_library(path: str = LIB_PATH):
    """Load libpkv.so (once). Raises if it is missing: build it with
    ``python -m paged_kv_attention_28_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpkv.so not found at {path}; build it with "
                           "`python -m paged_kv_attention_28_amd.build` (no fallback path exists)")
    lib = ctypes.CDLL(path)
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_abi_version.restype = c_i32
    lib.pkv_abi_version.argtypes = []
    lib.pkv_prepare_step.restype = c_i32
    lib.pkv_prepare_step.argtypes = [c_i32, P_I32, P_I32, P_I32, P_I64, c_i32, c_i32, c_i32, P_I32, c_i64,
                                     P_I32, P_I32, P_I32, P_I64, P_I32, P_I32]
    lib.kv_store.restype = c_i32
    lib.kv_store.argtypes = [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_i64, c_vp]
    lib.paged_attn_decode_workspace_size.restype = c_size
    lib.paged_attn_decode_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32]
    lib.paged_attn_decode.restype = c_i32
    lib.paged_attn_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                      c_i64, c_f32, c_i32, c_vp, c_size, c_vp]
    lib.paged_attn_decode_noalloc.restype = c_i32
    lib.paged_attn_decode_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32,
                                              c_i32, c_i64, c_f32, c_i32, c_vp]
    lib.paged_attn_decode_store.restype = c_i32
    lib.paged_attn_decode_store.argtypes = [c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp,
                                            c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_f32, c_i32, c_vp, c_size,
                                            c_vp]
    lib.paged_attn_prefill_varlen.restype = c_i32
    lib.paged_attn_prefill_varlen.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                              c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_f32, c_vp, c_i32,
                                              c_vp]
    lib.paged_attn_prefill_store.restype = c_i32
    lib.paged_attn_prefill_store.argtypes = [c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64,
                                             c_f32, c_vp, c_i32, c_vp]
    lib.pkv_prefill_plan.restype = c_i32
    lib.pkv_prefill_plan.argtypes = [c_i32, P_I32, P_I32, c_i32, c_i32, P_I32, c_i64, P_I64]
    lib.pkv_sched_create.restype = c_i32
    lib.pkv_sched_create.argtypes = [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]
    lib.pkv_sched_destroy.restype = c_i32
    lib.pkv_sched_destroy.argtypes = [c_vp]
    lib.pkv_sched_add.restype = c_i32
    lib.pkv_sched_add.argtypes = [c_vp, c_i32, c_i32, P_I32]
    lib.pkv_sched_schedule.restype = c_i32
    lib.pkv_sched_schedule.argtypes = [c_vp, ctypes.POINTER(SchedBatch)]
    lib.pkv_sched_postprocess.restype = c_i32
    lib.pkv_sched_postprocess.argtypes = [c_vp]
    lib.pkv_sched_unfinished.restype = c_i32
    lib.pkv_sched_unfinished.argtypes = [c_vp]
    lib.pkv_sched_free_blocks.restype = c_i32
    lib.pkv_sched_free_blocks.argtypes = [c_vp]
    lib.pkv_decode_graphs_create.restype = c_i32
    lib.pkv_decode_graphs_create.argtypes = [ctypes.POINTER(DecodeGraphDesc), P_I32, c_i32, ctypes.POINTER(c_vp)]
    lib.pkv_decode_graphs_create_layers.restype = c_i32
    lib.pkv_decode_graphs_create_layers.argtypes = [ctypes.POINTER(DecodeGraphDesc), c_i32, P_I32, c_i32,
                                                    ctypes.POINTER(c_vp)]
    lib.pkv_decode_graphs_launch.restype = c_i32
    lib.pkv_decode_graphs_launch.argtypes = [c_vp, c_i32, P_I32, c_vp]
    lib.pkv_decode_graphs_destroy.restype = c_i32
    lib.pkv_decode_graphs_destroy.argtypes = [c_vp]
    lib.rope_kv_store.restype = c_i32
    lib.rope_kv_store.argtypes = [c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_i64,
                                  c_i32, c_i32, c_i32, c_i32, c_i64, c_vp]
    lib.sample_temperature_workspace_size.restype = c_size
    lib.sample_temperature_workspace_size.argtypes = [c_i32, c_i32]
    lib.sample_temperature.restype = c_i32
    lib.sample_temperature.argtypes = [c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_i32, c_i32, c_vp, c_size, c_vp]
    lib.pkv_rope_cos_sin.restype = c_i32
    lib.pkv_rope_cos_sin.argtypes = [ctypes.POINTER(ctypes.c_float), c_i32, c_i32, ctypes.c_double]
    if lib.pkv_abi_version() != ABI_VERSION:
        raise RuntimeError("libpkv.so ABI version mismatch")
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != PKV_OK:
        raise PkvError(fn, status, _lib.pkv_last_error().decode())


def last_error() -> str:
    return load_library().pkv_last_error().decode()


# ----------------------------------------------------------------------------
# host: step preparation
# ----------------------------------------------------------------------------

def _i32p(a: np.ndarray):
    return a.ctypes.data_as(P_I32)


class StepMeta:
    """Host metadata of one step, as built by ``pkv_prepare_step``."""

    def __init__(self, slot_mapping, cu_seqlens_q, context_lens, block_tables, num_tokens, max_q_len,
                 max_context_len):
        self.slot_mapping = slot_mapping
        self.cu_seqlens_q = cu_seqlens_q
        self.context_lens = context_lens
        self.block_tables = block_tables
        self.num_tokens = num_tokens
        self.max_q_len = max_q_len
        self.max_context_len = max_context_len


def pkv_prepare_step(seq_lens, num_cached, block_tables, block_size: int, max_blocks_per_seq: int,
                     num_pad: int = 0, out=None) -> StepMeta:
    """Call ``pkv_prepare_step`` on host arrays. ``block_tables`` is a list of
    per-sequence lists of block ids. ``out`` may hold preallocated host
    (e.g. pinned) numpy arrays to write into."""
    lib = load_library()
    S = len(seq_lens)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    num_cached = np.ascontiguousarray(num_cached, dtype=np.int32)
    offs = np.zeros(S + 1, dtype=np.int64)
    if S:
        offs[1:] = np.cumsum([len(t) for t in block_tables])
    data = (np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32) for t in block_tables]))
            if S and offs[-1] else np.zeros(1, dtype=np.int32))
    rows = S + num_pad
    cap = int((seq_lens.astype(np.int64) - num_cached).sum()) + num_pad if S else num_pad
    if out is None:
        slots = np.empty(max(cap, 1), dtype=np.int32)
        cu = np.empty(rows + 1, dtype=np.int32)
        ctx = np.empty(max(rows, 1), dtype=np.int32)
        bt = np.empty(max(rows * max_blocks_per_seq, 1), dtype=np.int32)
    else:
        slots, cu, ctx, bt = out
        cap = slots.size
    nt, mq, mc = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.pkv_prepare_step(S, _i32p(seq_lens), _i32p(num_cached), _i32p(data), offs.ctypes.data_as(P_I64),
                              int(num_pad), int(block_size), int(max_blocks_per_seq), _i32p(slots), int(cap),
                              _i32p(cu), _i32p(ctx), _i32p(bt), ctypes.byref(nt), ctypes.byref(mq),
                              ctypes.byref(mc))
    _check("pkv_prepare_step", st)
    n = nt.value
    return StepMeta(slots[:n], cu[:rows + 1], ctx[:rows], bt[:rows * max_blocks_per_seq].reshape(rows, max_blocks_per_seq),
                    n, mq.value, mc.value)


class StepPrep:
    """``pkv_prepare_step`` (and, for a prefill step, ``pkv_prefill_plan``)
    on a sequence state held as arrays, the form a scheduler keeps it in
    (``pkv_sched_batch`` hands out the same CSR arrays): the arrays and the
    calls' pointer arguments are built once, so each call costs one C call
    per function writing into ``out`` (e.g. pinned buffers). Calling it
    again recomputes the metadata from the (possibly updated) arrays
    ``seq_lens``, ``num_cached`` and ``bt_data``."""

    def __init__(self, seq_lens, num_cached, block_tables, block_size: int, max_blocks_per_seq: int,
                 num_pad: int, out, plan_heads=None, plan_out=None):
        self.lib = load_library()
        S = len(seq_lens)
        self.seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        self.num_cached = np.ascontiguousarray(num_cached, dtype=np.int32)
        self.bt_offsets = np.zeros(S + 1, dtype=np.int64)
        if S:
            self.bt_offsets[1:] = np.cumsum([len(t) for t in block_tables])
        self.bt_data = (np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32) for t in block_tables]))
                        if S and self.bt_offsets[-1] else np.zeros(1, dtype=np.int32))
        self.rows = S + num_pad
        self.mb = max_blocks_per_seq
        self.out = out
        slots, cu, ctx, bt = out
        for a in out:
            if a.dtype != np.int32 or not a.flags.c_contiguous:
                raise ValueError("out arrays must be contiguous int32")
        self._nt, self._mq, self._mc = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0)
        self._args = (S, _i32p(self.seq_lens), _i32p(self.num_cached), _i32p(self.bt_data),
                      self.bt_offsets.ctypes.data_as(P_I64), int(num_pad), int(block_size), int(max_blocks_per_seq),
                      _i32p(slots), int(slots.size), _i32p(cu), _i32p(ctx), _i32p(bt), ctypes.byref(self._nt),
                      ctypes.byref(self._mq), ctypes.byref(self._mc))
        self.plan_out = plan_out
        self._n_items = ctypes.c_int64(0)
        if plan_heads is not None:
            if plan_out.dtype != np.int32 or not plan_out.flags.c_contiguous:
                raise ValueError("plan_out must be a contiguous int32 array")
            self._plan_args = (self.rows, _i32p(cu), _i32p(ctx), int(plan_heads[0]), int(plan_heads[1]),
                               _i32p(plan_out), plan_out.size // 2, ctypes.byref(self._n_items))
        else:
            self._plan_args = None

    def __call__(self):
        """Returns (StepMeta, number of plan items or 0)."""
        _check("pkv_prepare_step", self.lib.pkv_prepare_step(*self._args))
        slots, cu, ctx, bt = self.out
        n = self._nt.value
        m = StepMeta(slots[:n], cu[:self.rows + 1], ctx[:self.rows],
                     bt[:self.rows * self.mb].reshape(self.rows, self.mb), n, self._mq.value, self._mc.value)
        items = 0
        if self._plan_args is not None:
            _check("pkv_prefill_plan", self.lib.pkv_prefill_plan(*self._plan_args))
            items = self._n_items.value
        return m, items


def pkv_prefill_plan(cu_seqlens_q, context_lens, num_q_heads: int, num_kv_heads: int, out=None) -> np.ndarray:
    """Call ``pkv_prefill_plan`` on host arrays; returns int32 [n, 2] items.
    ``out`` may be a preallocated host int32 array of 2 * capacity elements
    (e.g. a pinned buffer); the result is then a view of it."""
    lib = load_library()
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = cu.size - 1
    if S < 0 or ctx.size < S:
        raise ValueError("cu_seqlens_q / context_lens do not describe a batch")
    n = ctypes.c_int64(0)
    if out is None:
        st = lib.pkv_prefill_plan(S, _i32p(cu), _i32p(ctx), int(num_q_heads), int(num_kv_heads), None, 0,
                                  ctypes.byref(n))
        _check("pkv_prefill_plan", st)
        out = np.empty(max(2 * n.value, 2), dtype=np.int32)
    if out.dtype != np.int32 or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous int32 array")
    st = lib.pkv_prefill_plan(S, _i32p(cu), _i32p(ctx), int(num_q_heads), int(num_kv_heads), _i32p(out),
                              out.size // 2, ctypes.byref(n))
    _check("pkv_prefill_plan", st)
    return out[:2 * n.value].reshape(n.value, 2)


def prefill_plan_capacity(total_q: int, num_seqs: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Upper bound on the plan's item count for any batch of ``num_seqs``
    sequences with ``total_q`` query tokens in all."""
    tok = 128 // (num_q_heads // num_kv_heads)
    return num_kv_heads * (total_q // tok + num_seqs)


class SchedStep:
    """One scheduled step, copied out of the scheduler's buffers."""

    def __init__(self, kind, request_ids, seq_lens, num_cached, full_lens, block_tables, num_pad, chunked_first,
                 preempted):
        self.kind = kind                    # "prefill" or "decode"
        self.request_ids = request_ids      # list of int
        self.seq_lens = seq_lens
        self.num_cached = num_cached
        self.full_lens = full_lens
        self.block_tables = block_tables    # list of lists of block ids
        self.num_pad = num_pad
        self.chunked_first = chunked_first
        self.preempted = preempted


class Scheduler:
    """The native scheduler (``pkv_sched_*``): add requests, then
    ``schedule()`` / ``postprocess()`` until ``schedule()`` returns None."""

    def __init__(self, num_blocks: int, block_size: int, max_num_seqs: int, max_num_batched_tokens: int):
        self._lib = load_library()
        h = c_vp()
        _check("pkv_sched_create", self._lib.pkv_sched_create(int(num_blocks), int(block_size), int(max_num_seqs),
                                                              int(max_num_batched_tokens), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            self._lib.pkv_sched_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, prompt_len: int, output_len: int) -> int:
        rid = ctypes.c_int32(-1)
        _check("pkv_sched_add", self._lib.pkv_sched_add(self._h, int(prompt_len), int(output_len), ctypes.byref(rid)))
        return rid.value

    def schedule(self):
        b = SchedBatch()
        _check("pkv_sched_schedule", self._lib.pkv_sched_schedule(self._h, ctypes.byref(b)))
        if b.kind < 0:
            return None
        n = b.num_seqs
        off = [b.bt_offsets[i] for i in range(n + 1)]
        return SchedStep("prefill" if b.kind == 1 else "decode", [b.request_ids[i] for i in range(n)],
                         [b.seq_lens[i] for i in range(n)], [b.num_cached[i] for i in range(n)],
                         [b.full_lens[i] for i in range(n)],
                         [[b.bt_data[j] for j in range(off[i], off[i + 1])] for i in range(n)], b.num_pad,
                         bool(b.chunked_first), [b.preempted[i] for i in range(b.num_preempted)])

    def postprocess(self):
        _check("pkv_sched_postprocess", self._lib.pkv_sched_postprocess(self._h))

    @property
    def unfinished(self) -> int:
        return self._lib.pkv_sched_unfinished(self._h)

    @property
    def free_blocks(self) -> int:
        return self._lib.pkv_sched_free_blocks(self._h)

    def run(self, prompts, outputs):
        """Add the requests and run the schedule to completion; the list of steps."""
        for p, o in zip(prompts, outputs):
            self.add(p, o)
        steps = []
        while True:
            st = self.schedule()
            if st is None:
                return steps
            steps.append(st)
            self.postprocess()


# ----------------------------------------------------------------------------
# device calls
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    """Raw HIP stream handle: `stream`'s, else the current device's current
    stream (read through torch's raw-handle getter where the build has it:
    building a Stream object costs about 2.5 us of host time per call)."""
    torch = _torch()
    if stream is not None:
        return int(stream.cuda_stream)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(torch.cuda.current_device()))
    return int(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype, contiguous=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def kv_store(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """key/value [T, H_kv, D] bf16 (token stride may exceed a row); caches
    [N, 256, H_kv, 128] bf16; slot_mapping [T] int32."""
    torch = _torch()
    lib = load_library()
    T = key.shape[0]
    if value.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("key, value and slot_mapping must have the same number of tokens")
    for t, n in ((key, "key"), (value, "value")):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{n} rows must be contiguous [H_kv, D]")
    N, B, H, D = k_cache.shape
    st = lib.kv_store(_dev(key, "key", torch.bfloat16, False), key.stride(0),
                      _dev(value, "value", torch.bfloat16, False), value.stride(0),
                      _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
                      _dev(slot_mapping, "slot_mapping", torch.int32), T, H, D, B, N, _stream(stream))
    _check("kv_store", st)


def pkv_rope_cos_sin(max_position: int, head_dim: int = 128, theta: float = 1.0e6) -> np.ndarray:
    """Host float32 [max_position, head_dim] table: cos of each pair's angle,
    then its sine (``pkv_rope_cos_sin``)."""
    lib = load_library()
    out = np.empty((int(max_position), int(head_dim)), dtype=np.float32)
    _check("pkv_rope_cos_sin", lib.pkv_rope_cos_sin(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                                     int(max_position), int(head_dim), float(theta)))
    return out


def rope_kv_store(q, key, value, positions, cos_sin, k_cache, v_cache, slot_mapping, stream=None):
    """q [T, H_q, D] bf16 (rotated in place; token stride may exceed a row);
    key/value [T, H_kv, D] bf16; positions, slot_mapping [T] int32; cos_sin
    [max_position, D] float32 device table; caches [N, 256, H_kv, 128]."""
    torch = _torch()
    lib = load_library()
    T = q.shape[0]
    if key.shape[0] != T or value.shape[0] != T or slot_mapping.shape[0] != T or positions.shape[0] != T:
        raise ValueError("q, key, value, positions and slot_mapping must have the same number of tokens")
    for t, n in ((q, "q"), (key, "key"), (value, "value")):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{n} rows must be contiguous [H, D]")
    N, B, H, D = k_cache.shape
    st = lib.rope_kv_store(_dev(q, "q", torch.bfloat16, False), q.stride(0), _dev(key, "key", torch.bfloat16, False),
                           key.stride(0), _dev(value, "value", torch.bfloat16, False), value.stride(0),
                           _dev(positions, "positions", torch.int32), _dev(cos_sin, "cos_sin", torch.float32),
                           cos_sin.shape[0], _dev(k_cache, "k_cache", torch.bfloat16),
                           _dev(v_cache, "v_cache", torch.bfloat16), _dev(slot_mapping, "slot_mapping", torch.int32),
                           T, q.shape[1], H, D, B, N, _stream(stream))
    _check("rope_kv_store", st)


def sample_temperature_workspace_size(num_rows: int, vocab: int) -> int:
    return int(load_library().sample_temperature_workspace_size(int(num_rows), int(vocab)))


def sample_temperature(out_tokens, logits, temperatures, gumbel, workspace=None, stream=None):
    """out_tokens [R] int32; logits, gumbel [R, V] float32 (row stride may
    exceed V); temperatures [R] float32; workspace uint8 (allocated if None)."""
    torch = _torch()
    lib = load_library()
    R, V = logits.shape
    if gumbel.shape != logits.shape or temperatures.shape[0] != R or out_tokens.shape[0] != R:
        raise ValueError("shapes of logits, gumbel, temperatures and out_tokens do not match")
    for t, n in ((logits, "logits"), (gumbel, "gumbel")):
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if workspace is None:
        workspace = torch.empty(max(sample_temperature_workspace_size(R, V), 16), dtype=torch.uint8,
                                device=logits.device)
    st = lib.sample_temperature(_dev(out_tokens, "out_tokens", torch.int32), _dev(logits, "logits", torch.float32, False),
                                logits.stride(0), _dev(temperatures, "temperatures", torch.float32),
                                _dev(gumbel, "gumbel", torch.float32, False), gumbel.stride(0), R, V,
                                _dev(workspace, "workspace", workspace.dtype),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("sample_temperature", st)


def paged_attn_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len) -> int:
    return int(load_library().paged_attn_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                               max_context_len))


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                      workspace=None, stream=None):
    """out/q [S, H_q, D] bf16; block_tables [S, stride] int32; context_lens [S] int32."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] < S or context_lens.shape[0] < S:
        raise ValueError("block_tables / context_lens do not cover the batch")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", workspace.dtype)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.paged_attn_decode(_dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
                               _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
                               _dev(block_tables, "block_tables", torch.int32), block_tables.stride(0),
                               _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, N,
                               float(scale), int(max_context_len), ws_ptr, ws_bytes, _stream(stream))
    _check("paged_attn_decode", st)


def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                              stream=None):
    """paged_attn_decode on the library's own scratch array (no workspace argument); same arguments otherwise."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] < S or context_lens.shape[0] < S:
        raise ValueError("block_tables / context_lens do not cover the batch")
    st = lib.paged_attn_decode_noalloc(_dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
                                       _dev(k_cache, "k_cache", torch.bfloat16),
                                       _dev(v_cache, "v_cache", torch.bfloat16),
                                       _dev(block_tables, "block_tables", torch.int32), block_tables.stride(0),
                                       _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, N,
                                       float(scale), int(max_context_len), _stream(stream))
    _check("paged_attn_decode_noalloc", st)


def paged_attn_decode_store(out, q, key, value, slot_mapping, k_cache, v_cache, block_tables, context_lens, scale,
                            max_context_len, workspace=None, stream=None):
    """kv_store of the new tokens and paged_attn_decode in one call. key/value
    [S, H_kv, D] bf16 (row s: sequence s's new token, token stride may exceed
    a row); slot_mapping [S] int32 (cache row of position context_lens[s] - 1,
    -1 for padding rows); the rest as for paged_attn_decode."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] < S or context_lens.shape[0] < S:
        raise ValueError("block_tables / context_lens do not cover the batch")
    if key.shape[0] < S or value.shape[0] < S or slot_mapping.shape[0] < S:
        raise ValueError("key, value and slot_mapping must cover the batch")
    for t, n in ((key, "key"), (value, "value")):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{n} rows must be contiguous [H_kv, D]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", workspace.dtype)
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.paged_attn_decode_store(_dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
                                     _dev(key, "key", torch.bfloat16, False), key.stride(0),
                                     _dev(value, "value", torch.bfloat16, False), value.stride(0),
                                     _dev(slot_mapping, "slot_mapping", torch.int32),
                                     _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
                                     _dev(block_tables, "block_tables", torch.int32), block_tables.stride(0),
                                     _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D, B, N,
                                     float(scale), int(max_context_len), ws_ptr, ws_bytes, _stream(stream))
    _check("paged_attn_decode_store", st)


def paged_attn_prefill_varlen(out, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables, max_q_len,
                              max_context_len, scale, work_items=None, stream=None):
    """out/q [T, H_q, D] bf16; cu_seqlens_q [S+1]; context_lens [S];
    block_tables [S, stride] int32; work_items: device int32 [n, 2] from
    ``pkv_prefill_plan`` for the same batch, or None for the full grid."""
    torch = _torch()
    lib = load_library()
    T, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] < S or context_lens.shape[0] < S:
        raise ValueError("block_tables / context_lens do not cover the batch")
    wi_ptr, wi_n = None, 0
    if work_items is not None:
        if work_items.dim() != 2 or work_items.shape[1] != 2:
            raise ValueError("work_items must be [n, 2]")
        wi_ptr, wi_n = _dev(work_items, "work_items", torch.int32), work_items.shape[0]
    st = lib.paged_attn_prefill_varlen(_dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
                                       _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                                       _dev(context_lens, "context_lens", torch.int32),
                                       _dev(k_cache, "k_cache", torch.bfloat16),
                                       _dev(v_cache, "v_cache", torch.bfloat16),
                                       _dev(block_tables, "block_tables", torch.int32), block_tables.stride(0), S,
                                       T, int(max_q_len), int(max_context_len), Hq, Hkv, D, B, N, float(scale),
                                       wi_ptr, int(wi_n), _stream(stream))
    _check("paged_attn_prefill_varlen", st)


def paged_attn_prefill_store(out, q, key, value, slot_mapping, k_cache, v_cache, cu_seqlens_q, context_lens,
                             block_tables, max_q_len, max_context_len, scale, work_items=None, stream=None):
    """kv_store of the step's tokens and paged_attn_prefill_varlen in one call. key/value [T, H_kv, D] bf16 (token
    stride may exceed a row); slot_mapping [T] int32; the rest as for paged_attn_prefill_varlen."""
    torch = _torch()
    lib = load_library()
    T, Hq, D = q.shape
    N, B, Hkv, _ = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] < S or context_lens.shape[0] < S:
        raise ValueError("block_tables / context_lens do not cover the batch")
    if key.shape[0] < T or value.shape[0] < T or slot_mapping.shape[0] < T:
        raise ValueError("key, value and slot_mapping must cover the step's tokens")
    for t, n in ((key, "key"), (value, "value")):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{n} rows must be contiguous [H_kv, D]")
    wi_ptr, wi_n = None, 0
    if work_items is not None:
        if work_items.dim() != 2 or work_items.shape[1] != 2:
            raise ValueError("work_items must be [n, 2]")
        wi_ptr, wi_n = _dev(work_items, "work_items", torch.int32), work_items.shape[0]
    st = lib.paged_attn_prefill_store(_dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
                                      _dev(key, "key", torch.bfloat16, False), key.stride(0),
                                      _dev(value, "value", torch.bfloat16, False), value.stride(0),
                                      _dev(slot_mapping, "slot_mapping", torch.int32),
                                      _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
                                      _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                                      _dev(context_lens, "context_lens", torch.int32),
                                      _dev(block_tables, "block_tables", torch.int32), block_tables.stride(0), S, T,
                                      int(max_q_len), int(max_context_len), Hq, Hkv, D, B, N, float(scale), wi_ptr,
                                      int(wi_n), _stream(stream))
    _check("paged_attn_prefill_store", st)


def _graph_desc(key, value, slot_mapping, k_cache, v_cache, q, out, block_tables, context_lens, workspace, scale,
                max_context_len, rows):
    torch = _torch()
    N, B, Hkv, D = k_cache.shape
    d = DecodeGraphDesc()
    d.key = _dev(key, "key", torch.bfloat16, False)
    d.key_stride = key.stride(0)
    d.value = _dev(value, "value", torch.bfloat16, False)
    d.value_stride = value.stride(0)
    d.slot_mapping = _dev(slot_mapping, "slot_mapping", torch.int32)
    d.k_cache = _dev(k_cache, "k_cache", torch.bfloat16)
    d.v_cache = _dev(v_cache, "v_cache", torch.bfloat16)
    d.num_blocks = N
    d.q = _dev(q, "q", torch.bfloat16)
    d.out = _dev(out, "out", torch.bfloat16)
    d.block_tables = _dev(block_tables, "block_tables", torch.int32)
    d.block_table_stride = block_tables.stride(0)
    d.context_lens = _dev(context_lens, "context_lens", torch.int32)
    d.workspace = _dev(workspace, "workspace", workspace.dtype)
    d.workspace_bytes = workspace.numel() * workspace.element_size()
    d.num_q_heads, d.num_kv_heads, d.head_dim, d.block_size = q.shape[1], Hkv, D, B
    d.scale = float(scale)
    d.max_context_len = int(max_context_len)
    for t, nm in ((key, "key"), (value, "value"), (slot_mapping, "slot_mapping"), (q, "q"), (out, "out"),
                  (block_tables, "block_tables"), (context_lens, "context_lens")):
        if t.shape[0] < rows:
            raise ValueError(f"{nm} has {t.shape[0]} rows, the largest bucket needs {rows}")
    return d


class DecodeGraphs:
    """Decode-step graphs (``pkv_decode_graphs_*``) over static device
    buffers: key/value [rows, H_kv, D], slot_mapping [rows], q/out
    [rows, H_q, D], block_tables [rows, stride], context_lens [rows] and a
    workspace sized for the largest bucket. The tensors are kept alive with
    the handle; fill rows [0, batch), pad the rest up to the bucket (slot -1,
    context 0) and call ``launch(batch)``. ``layers`` (optional) lists further
    layers as (key, value, k_cache, v_cache, q, out) tuples sharing the
    metadata and the workspace; each replay then runs every layer in order
    (``pkv_decode_graphs_create_layers``)."""

    def __init__(self, key, value, slot_mapping, k_cache, v_cache, q, out, block_tables, context_lens, workspace,
                 scale, max_context_len, buckets, layers=()):
        self._lib = load_library()
        self.buckets = sorted(int(b) for b in buckets)
        rows = max(self.buckets)
        all_layers = [(key, value, k_cache, v_cache, q, out)] + list(layers)
        self._keep = (all_layers, slot_mapping, block_tables, context_lens, workspace)
        descs = (DecodeGraphDesc * len(all_layers))()
        for i, (k, v, kc, vc, qq, oo) in enumerate(all_layers):
            descs[i] = _graph_desc(k, v, slot_mapping, kc, vc, qq, oo, block_tables, context_lens, workspace, scale,
                                   max_context_len, rows)
        arr = (ctypes.c_int32 * len(self.buckets))(*self.buckets)
        h = c_vp()
        _check("pkv_decode_graphs_create",
               self._lib.pkv_decode_graphs_create_layers(descs, len(all_layers), arr, len(self.buckets),
                                                         ctypes.byref(h)))
        self._h = h

    def launch(self, batch: int, stream=None) -> int:
        """Replay the smallest bucket >= batch; returns that bucket."""
        b = ctypes.c_int32(0)
        _check("pkv_decode_graphs_launch", self._lib.pkv_decode_graphs_launch(self._h, int(batch), ctypes.byref(b),
                                                                              _stream(stream)))
        return b.value

    def close(self):
        if self._h:
            self._lib.pkv_decode_graphs_destroy(self._h)
            self._h = c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
