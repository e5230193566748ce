"""fp64 oracle for the rotary position embedding applied before the KV store.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and
the CPU-baseline leg of the benchmark may call this module.

P2 = "读 Nano-vLLM 源码：一个极简 LLM 推理引擎是如何工作的": in its attention
layer sketch the query and key projections get the rotary position encoding
(rotary_emb(q, k, positions)) before K and V are written to the cache blocks
and attention reads them back; the engine's layer list has a rotary_embedding
module. The pages give no formula.

Reading (parity unpinned by the pages; a convention of the model family the
workload shapes come from): the "rotate half" form. For a head vector x of
even length D, pair element i with element i + D/2 (i < D/2) and rotate the
pair by the angle  pos * theta ** (-2 i / D):
    y[i]       = x[i] cos a_i - x[i + D/2] sin a_i
    y[i + D/2] = x[i + D/2] cos a_i + x[i] sin a_i
with theta = 1e6 by default. Every head (query and key) uses the same angles;
values are not rotated. Pins (tests/test_rope.py): position 0 is the
identity; each pair keeps its norm; rotations compose (positions add); the
product of a rotated query and a rotated key depends only on the position
difference; D = 2 is the plain 2-d rotation by pos radians; unit vectors turn
by angles worked out by hand for theta = 10^4, D = 8 (pair i at 10^-i rad per
position) and for theta = 10^6, D = 128 (pairs 0 and 32), which pins the
frequency schedule (tests/golden/rope_angles_closed_form.json).
"""

from __future__ import annotations

import numpy as np

from .paged import bf16_bits_to_f64

DEFAULT_THETA = 1.0e6


def rope_angles(positions, head_dim: int, theta: float = DEFAULT_THETA) -> np.ndarray:
    """[n, head_dim / 2] angles pos * theta^(-2 i / head_dim), fp64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope_ref(x, positions, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotate x [n, H, D] (fp64 values, or bf16 bit patterns as uint16) at
    the given positions; returns fp64 [n, H, D]."""
    x = bf16_bits_to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    n, H, D = x.shape
    a = rope_angles(positions, D, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 to bf16 (nearest, ties to even) and return the bit patterns.

    The value is first rounded to fp32 (exact for every result of interest
    here up to one fp32 rounding), then its 32-bit pattern is rounded to the
    upper 16 bits with ties to even."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def rope_kv_store_ref(q_bits, k_bits, v_bits, positions, slot_mapping, k_cache, v_cache,
                      theta: float = DEFAULT_THETA):
    """The fused step on copies of the caches: rotate q and k, store rotated
    K (rounded to bf16) and V (bit copy) at the slots (-1 skipped).

    Returns (q_rot fp64 [n, H_q, D], k_rot fp64 [n, H_kv, D], new k_cache,
    new v_cache)."""
    from .paged import kv_store_ref
    q_rot = rope_ref(q_bits, positions, theta)
    k_rot = rope_ref(k_bits, positions, theta)
    kc, vc = kv_store_ref(k_cache, v_cache, f64_to_bf16_bits(k_rot), v_bits, slot_mapping)
    return q_rot, k_rot, kc, vc
