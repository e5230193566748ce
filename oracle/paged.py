"""fp64 numpy oracle: per-step metadata, KV store, paged decode and prefill attention.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and
the CPU-baseline leg of the benchmark may call this module.

Page references:
  P1 = "13. 读一个最小推理引擎：nano-vllm"
  P2 = "读 Nano-vLLM 源码：一个极简 LLM 推理引擎是如何工作的"

Arrays holding bf16 data are passed as ``numpy.uint16`` bit patterns so that the
store is checked as a bit copy and the attention inputs are widened to fp64
exactly (a bf16 value is the top half of an fp32 value).

Cache layout (one layer): ``cache[num_blocks, block_size, H_kv, D]``. The pages
allocate one tensor shaped (2, layers, blocks, block_size, H_kv, D) once and
never reallocate it (P1, "第五站：执行准备与 KV 容量"); one layer's K or V is the
4-d slice used here.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "prepare_step_ref",
    "kv_store_ref",
    "kv_store_inplace_ref",
    "gather_context_ref",
    "attn_contiguous_ref",
    "decode_ref",
    "prefill_ref",
]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    a = np.asarray(bits)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    wide = a.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# a1: per-step metadata
# ----------------------------------------------------------------------------

def _physical_slot(table, pos: int, block_size: int) -> int:
    """Slot of logical position ``pos``: table[pos // bs] * bs + pos % bs.

    P1, "第五站：执行准备与 KV 容量": a token's K/V goes to the row given by the
    block table entry of its logical block times the block size plus its
    offset inside the block.
    """
    return int(table[pos // block_size]) * block_size + pos % block_size


def prepare_step_ref(seq_lens, num_cached, block_tables, block_size: int,
                     max_blocks_per_seq: int, num_pad: int = 0):
    """Metadata for one engine step, as the step preparation builds it.

    Inputs, per real sequence b: ``seq_lens[b]`` = len(seq) after this step's
    tokens are appended, ``num_cached[b]`` = tokens already in the cache,
    ``block_tables[b]`` = list of physical block ids.

    P1, "第二站：一个请求的状态": the step computes tokens from num_cached onward,
    one field covering prefix hits, chunk continuations and decode.
    P1, "第五站：执行准备与 KV 容量": prefill feeds only tokens from num_cached
    onward; slot_mapping holds one slot per computed token.
    Decode is the case seq_len - num_cached == 1 (the new token at len - 1).
    P1, same section (CUDA Graph paragraph): padding rows of a replayed batch
    get slot -1. Reading: each padding row is one token with context length 0
    and an all -1 block-table row.

    Returns (slot_mapping[int32 T], cu_seqlens_q[int32 S+P+1],
    context_lens[int32 S+P], block_tables[int32 (S+P) x max_blocks_per_seq]).
    """
    S = len(seq_lens)
    slots: list[int] = []
    cu = [0]
    ctx: list[int] = []
    bt = np.full((S + num_pad, max_blocks_per_seq), -1, dtype=np.int32)
    for b in range(S):
        L = int(seq_lens[b])
        c = int(num_cached[b])
        table = list(block_tables[b])
        if not (0 <= c < L):
            raise ValueError(f"seq {b}: need 0 <= num_cached < seq_len, got {c}, {L}")
        needed = -(-L // block_size)
        if len(table) < needed or len(table) > max_blocks_per_seq:
            raise ValueError(f"seq {b}: block table has {len(table)} entries, needs {needed}")
        for pos in range(c, L):
            slots.append(_physical_slot(table, pos, block_size))
        cu.append(cu[-1] + (L - c))
        ctx.append(L)
        bt[b, : len(table)] = table
    for _ in range(num_pad):
        slots.append(-1)
        cu.append(cu[-1] + 1)
        ctx.append(0)
    return (np.asarray(slots, dtype=np.int32), np.asarray(cu, dtype=np.int32),
            np.asarray(ctx, dtype=np.int32), bt)


# ----------------------------------------------------------------------------
# a2: KV store
# ----------------------------------------------------------------------------

def kv_store_inplace_ref(k_cache, v_cache, key, value, slot_mapping) -> None:
    """Copy token rows into the paged cache arrays in place (uint16 arrays).

    P1, "第六站：注意力层": one program per token reads its slot, returns early
    when the slot is -1, and copies the token's whole K row and V row (all KV
    heads, token stride given by the key/value tensors) to row ``slot`` of the
    flattened cache. Rows are copied bit for bit.

    Readings: a slot outside [0, num_blocks * block_size) other than -1 is a
    caller error (raises); two tokens may not name the same slot in one call
    (raises), since the result would depend on write order. Nothing is
    written when an error is raised.
    """
    if k_cache.dtype != np.uint16 or v_cache.dtype != np.uint16:
        raise TypeError("caches must be uint16 bit patterns")
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous to be written in place")
    N, B, H, D = k_cache.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    key = np.asarray(key, dtype=np.uint16).reshape(len(slots), H, D)
    value = np.asarray(value, dtype=np.uint16).reshape(len(slots), H, D)
    live = slots != -1
    s = slots[live]
    if s.size:
        if s.min() < 0 or s.max() >= N * B:
            raise ValueError("slot out of range")
        if np.unique(s).size != s.size:
            raise ValueError("duplicate slot in one store")
    k_cache.reshape(N * B, H, D)[s] = key[live]
    v_cache.reshape(N * B, H, D)[s] = value[live]


def kv_store_ref(k_cache, v_cache, key, value, slot_mapping):
    """The store on copies of the caches; returns the new (k_cache, v_cache)."""
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    kv_store_inplace_ref(kc, vc, key, value, slot_mapping)
    return kc, vc


# ----------------------------------------------------------------------------
# gather + attention
# ----------------------------------------------------------------------------

def _logical_to_physical(table_row, L: int, block_size: int) -> np.ndarray:
    """Physical row of each logical position 0..L-1 through one block table."""
    pos = np.arange(L, dtype=np.int64)
    table = np.asarray(table_row, dtype=np.int64)
    return table[pos // block_size] * block_size + pos % block_size


def gather_context_ref(cache, table_row, L: int) -> np.ndarray:
    """Rows of logical positions 0..L-1 of one sequence, shape [L, H_kv, D].

    P1, "第六站：注意力层": decode reads the history K/V from the paged cache
    through the block table, and a prefill with cached context passes the
    block table so the whole context is read from the cache.
    """
    N, B, H, D = cache.shape
    rows = _logical_to_physical(table_row, L, B)
    return np.asarray(cache).reshape(N * B, H, D)[rows]


def _kv_head_of(h: int, group: int) -> int:
    """KV head serving query head h. Reading: consecutive query heads share a
    KV head (h // group); the pages do not state the grouping."""
    return h // group


def _visible(q_pos, L: int) -> np.ndarray:
    """[n, L] mask: key j is visible to a query at absolute position p iff j <= p.

    Reading (bottom-right alignment): a query at absolute position p sees the
    cached prefix and the new tokens up to itself, which is what computing
    only the tokens from num_cached onward while reading the full context
    requires (P1, "第二站" and "第六站").
    """
    return np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]


def attn_contiguous_ref(q, K, V, q_pos, scale: float) -> np.ndarray:
    """Naive masked softmax attention on dense K/V; all fp64.

    q: [n, H_q, D]; K, V: [L, H_kv, D]; q_pos: [n] absolute positions.
    out[i, h] = sum_j softmax_j(scale * <q[i,h], K[j,g]>) V[j,g] over visible j,
    with g = _kv_head_of(h, H_q // H_kv).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, Hq, D = q.shape
    L, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    group = Hq // Hkv
    vis = _visible(q_pos, L)
    if n and not vis.any(axis=1).all():
        raise ValueError("a query row sees no key")
    out = np.zeros((n, Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = _kv_head_of(h, group)
        s = scale * (q[:, h, :] @ K[:, g, :].T)
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out


def decode_ref(q_bits, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """One query token per sequence at position len - 1; returns fp64 [S, H_q, D].

    P1, "第六站：注意力层": decode reads its history through the block table; the
    store runs first, so the context includes the current token.
    Reading: a row with context length 0 (a padding row) outputs zeros.
    """
    q = bf16_bits_to_f64(q_bits)
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for b in range(S):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = bf16_bits_to_f64(gather_context_ref(k_cache, block_tables[b], L))
        V = bf16_bits_to_f64(gather_context_ref(v_cache, block_tables[b], L))
        out[b] = attn_contiguous_ref(q[b:b + 1], K, V, [L - 1], scale)[0]
    return out


def prefill_ref(q_bits, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables,
                scale: float) -> np.ndarray:
    """Varlen causal prefill; queries of sequence b sit at positions c_b .. L_b - 1.

    n_b = cu[b+1] - cu[b] query tokens, L_b = context_lens[b], and
    c_b = L_b - n_b = num_cached_tokens (P1, "第二站": the step computes tokens
    from num_cached onward; "第六站": prefix-hit and chunk-continuation prefill
    read the whole context from the cache). Returns fp64 [sum n_b, H_q, D].
    """
    q = bf16_bits_to_f64(q_bits)
    T, Hq, D = q.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        L = int(context_lens[b])
        c = L - n
        if n <= 0:
            continue
        if c < 0:
            raise ValueError(f"seq {b}: context shorter than its query tokens")
        K = bf16_bits_to_f64(gather_context_ref(k_cache, block_tables[b], L))
        V = bf16_bits_to_f64(gather_context_ref(v_cache, block_tables[b], L))
        out[lo:hi] = attn_contiguous_ref(q[lo:hi], K, V, c + np.arange(n), scale)
    return out
