"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

No GPU. Each ``pin_*`` function raises when the oracle disagrees with a fact
that does not come from the oracle itself: a hand-derived fixture, a closed
form, an invariant, a scalar brute force, or torch's fp64 CPU
``scaled_dot_product_attention``. ``test_planted_mistakes`` plants plausible
mistakes in the oracle (on the CPU) and checks that some pin catches each.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import paged as op
from oracle.brute import brute_paged_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prepare_step_example.json")
NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# tiny random paged problems (generic block size, head dim and head counts)
# ----------------------------------------------------------------------------

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


class Problem:
    """Dense per-sequence K/V and queries, plus a shuffled paged pool that
    holds the same K/V (stored through the oracle's own prepare + store)."""

    def __init__(self, seed=0, B=4, D=8, Hq=4, Hkv=2, lens=(5, 9, 13), extra_blocks=3,
                 kv=None, q_scale=1.0):
        rng = np.random.default_rng(seed)
        self.B, self.D, self.Hq, self.Hkv = B, D, Hq, Hkv
        self.lens = list(lens)
        nb = [-(-L // B) for L in self.lens]
        self.N = sum(nb) + extra_blocks
        perm = [int(x) for x in rng.permutation(self.N)]
        self.tables, k = [], 0
        for n in nb:
            self.tables.append(perm[k:k + n])
            k += n
        self.mb = max(nb)
        if kv is None:
            self.K = [_bf16_bits(rng.standard_normal((L, Hkv, D))) for L in self.lens]
            self.V = [_bf16_bits(rng.standard_normal((L, Hkv, D))) for L in self.lens]
        else:
            self.K, self.V = kv(rng, self.lens, Hkv, D)
        self.qsrc = [_bf16_bits(q_scale * rng.standard_normal((L, Hq, D))) for L in self.lens]
        self.scale = 1.0 / math.sqrt(D)
        shape = (self.N, B, Hkv, D)
        kc = np.full(shape, NAN, dtype=np.uint16)
        vc = np.full(shape, NAN, dtype=np.uint16)
        slots, _, _, self.bt = op.prepare_step_ref(self.lens, [0] * len(self.lens), self.tables, B, self.mb)
        self.kc, self.vc = op.kv_store_ref(kc, vc, np.concatenate(self.K), np.concatenate(self.V), slots)

    def prefill(self, cached):
        """Queries for positions cached[b] .. L_b - 1 of every sequence."""
        qs = [self.qsrc[b][c:] for b, c in enumerate(cached)]
        cu = np.concatenate([[0], np.cumsum([len(x) for x in qs])]).astype(np.int32)
        ctx = np.asarray(self.lens, dtype=np.int32)
        return op.prefill_ref(np.concatenate(qs), cu, ctx, self.kc, self.vc, self.bt, self.scale)

    def decode(self):
        q = np.stack([self.qsrc[b][L - 1] for b, L in enumerate(self.lens)])
        ctx = np.asarray(self.lens, dtype=np.int32)
        return op.decode_ref(q, self.kc, self.vc, self.bt, ctx, self.scale)

    def dense(self, b):
        return (op.bf16_bits_to_f64(self.qsrc[b]), op.bf16_bits_to_f64(self.K[b]),
                op.bf16_bits_to_f64(self.V[b]))


def _rows(out, lens, cached):
    """Split a prefill output into per-sequence row blocks."""
    res, k = [], 0
    for L, c in zip(lens, cached):
        res.append(out[k:k + L - c])
        k += L - c
    return res


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_golden_prepare():
    """Hand-derived slot mapping / metadata from the pages' slot formula."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        slots, cu, ctx, bt = op.prepare_step_ref(c["seq_lens"], c["num_cached"], c["block_tables"],
                                                 c["block_size"], c["max_blocks_per_seq"], c["num_pad"])
        expect = []
        for first, count in c["expect_slot_runs"]:
            expect += [-1] * count if first == -1 else list(range(first, first + count))
        assert slots.tolist() == expect, c["name"]
        assert cu.tolist() == c["expect_cu_seqlens_q"], c["name"]
        assert ctx.tolist() == c["expect_context_lens"], c["name"]
        assert bt.tolist() == c["expect_block_tables"], c["name"]


def pin_store_rows():
    """Each live token's K/V row lands at (slot // B, slot % B) bit for bit
    (random bit patterns, NaN payloads included); every other row keeps its
    previous bits; -1 rows are skipped."""
    rng = np.random.default_rng(7)
    N, B, H, D = 5, 4, 2, 8
    kc = rng.integers(0, 1 << 16, size=(N, B, H, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(N, B, H, D), dtype=np.uint16)
    T = 12
    key = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint16)
    key[0, 0, 0] = 0x7FC1  # a NaN payload must survive
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int32)
    slots[[2, 5, 11]] = -1
    nk, nv = op.kv_store_ref(kc, vc, key, val, slots)
    written = set()
    for i, s in enumerate(slots):
        if s == -1:
            continue
        blk, off = divmod(int(s), B)
        assert np.array_equal(nk[blk, off], key[i]) and np.array_equal(nv[blk, off], val[i])
        written.add((blk, off))
    for blk in range(N):
        for off in range(B):
            if (blk, off) not in written:
                assert np.array_equal(nk[blk, off], kc[blk, off])
                assert np.array_equal(nv[blk, off], vc[blk, off])
    assert len(written) == T - 3


def pin_store_skip():
    """All -1 slots leave the cache untouched; duplicates and out-of-range
    slots are rejected."""
    rng = np.random.default_rng(8)
    kc = rng.integers(0, 1 << 16, size=(3, 4, 2, 8), dtype=np.uint16)
    vc = kc.copy()
    key = rng.integers(0, 1 << 16, size=(4, 2, 8), dtype=np.uint16)
    nk, nv = op.kv_store_ref(kc, vc, key, key, np.full(4, -1, np.int32))
    assert np.array_equal(nk, kc) and np.array_equal(nv, vc)
    for bad in ([0, 0, -1, -1], [12, -1, -1, -1], [-2, -1, -1, -1]):
        with pytest.raises(ValueError):
            op.kv_store_ref(kc, vc, key, key, np.asarray(bad, np.int32))


def pin_single_key():
    """A one-token context returns its V row exactly; so does prefill row 0
    of an uncached prompt."""
    pr = Problem(seed=1, lens=(1, 1, 6))
    out = pr.decode()
    G = pr.Hq // pr.Hkv
    for b in (0, 1):
        V = op.bf16_bits_to_f64(pr.V[b])
        for h in range(pr.Hq):
            assert np.array_equal(out[b, h], V[0, h // G])
    rows = _rows(pr.prefill([0, 0, 0]), pr.lens, [0, 0, 0])
    V2 = op.bf16_bits_to_f64(pr.V[2])
    for h in range(pr.Hq):
        assert np.array_equal(rows[2][0, h], V2[0, h // G])


def _same_keys(rng, lens, H, D):
    K, V = [], []
    for L in lens:
        row = rng.standard_normal((1, H, D))
        K.append(_bf16_bits(np.repeat(row, L, axis=0)))
        V.append(_bf16_bits(rng.standard_normal((L, H, D))))
    return K, V


def pin_identical_keys():
    """Identical keys give uniform weights: each row is the mean of the V rows
    it sees."""
    pr = Problem(seed=2, lens=(7, 11), kv=_same_keys)
    G = pr.Hq // pr.Hkv
    rows = _rows(pr.prefill([0, 3]), pr.lens, [0, 3])
    for b, c in enumerate([0, 3]):
        V = op.bf16_bits_to_f64(pr.V[b])
        for i in range(pr.lens[b] - c):
            p = c + i
            for h in range(pr.Hq):
                expect = V[:p + 1, h // G].mean(axis=0)
                np.testing.assert_allclose(rows[b][i, h], expect, rtol=1e-12, atol=1e-14)


def pin_zero_query():
    """A zero query also gives uniform weights (decode: mean of all V rows)."""
    pr = Problem(seed=3, lens=(9, 4), q_scale=0.0)
    out = pr.decode()
    G = pr.Hq // pr.Hkv
    for b, L in enumerate(pr.lens):
        V = op.bf16_bits_to_f64(pr.V[b])
        for h in range(pr.Hq):
            np.testing.assert_allclose(out[b, h], V[:L, h // G].mean(axis=0), rtol=1e-12, atol=1e-14)


def pin_two_keys_closed_form():
    """Two keys: out = (v0 + e^d v1) / (1 + e^d), d = scale (q.k1 - q.k0)."""
    pr = Problem(seed=4, lens=(2,))
    out = pr.decode()
    q, K, V = pr.dense(0)
    G = pr.Hq // pr.Hkv
    for h in range(pr.Hq):
        g = h // G
        d = pr.scale * (float(q[1, h] @ K[1, g]) - float(q[1, h] @ K[0, g]))
        e = math.exp(d)
        expect = (V[0, g] + e * V[1, g]) / (1.0 + e)
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-12, atol=1e-14)


def pin_convex_hull():
    """Every output lies within the per-dimension range of the V rows it sees."""
    pr = Problem(seed=5, lens=(13, 6, 9), q_scale=3.0)
    G = pr.Hq // pr.Hkv
    cached = [4, 0, 8]
    rows = _rows(pr.prefill(cached), pr.lens, cached)
    for b, c in enumerate(cached):
        V = op.bf16_bits_to_f64(pr.V[b])
        for i in range(pr.lens[b] - c):
            p = c + i
            for h in range(pr.Hq):
                lo = V[:p + 1, h // G].min(axis=0)
                hi = V[:p + 1, h // G].max(axis=0)
                assert np.all(rows[b][i, h] >= lo - 1e-12) and np.all(rows[b][i, h] <= hi + 1e-12)


def pin_permutation():
    """Relabelling physical blocks (pool and tables together) leaves every
    output bit-identical."""
    pr = Problem(seed=6, lens=(9, 13, 3))
    rng = np.random.default_rng(60)
    pi = rng.permutation(pr.N)
    kc2 = np.empty_like(pr.kc)
    vc2 = np.empty_like(pr.vc)
    kc2[pi] = pr.kc
    vc2[pi] = pr.vc
    bt2 = np.where(pr.bt >= 0, pi[np.maximum(pr.bt, 0)], -1).astype(np.int32)
    cached = [2, 5, 0]
    a = pr.prefill(cached)
    qs = [pr.qsrc[b][c:] for b, c in enumerate(cached)]
    cu = np.concatenate([[0], np.cumsum([len(x) for x in qs])]).astype(np.int32)
    b2 = op.prefill_ref(np.concatenate(qs), cu, np.asarray(pr.lens, np.int32), kc2, vc2, bt2, pr.scale)
    assert np.array_equal(a, b2)
    d1 = pr.decode()
    q = np.stack([pr.qsrc[b][L - 1] for b, L in enumerate(pr.lens)])
    d2 = op.decode_ref(q, kc2, vc2, bt2, np.asarray(pr.lens, np.int32), pr.scale)
    assert np.array_equal(d1, d2)


def pin_paged_equals_contiguous():
    """Reading through a shuffled block table equals attention on the dense K/V
    the pool was filled from, bit for bit."""
    pr = Problem(seed=9, lens=(9, 13, 4))
    cached = [3, 0, 1]
    rows = _rows(pr.prefill(cached), pr.lens, cached)
    for b, c in enumerate(cached):
        q, K, V = pr.dense(b)
        ref = op.attn_contiguous_ref(q[c:], K, V, c + np.arange(pr.lens[b] - c), pr.scale)
        assert np.array_equal(rows[b], ref)
    d = pr.decode()
    for b, L in enumerate(pr.lens):
        q, K, V = pr.dense(b)
        assert np.array_equal(d[b], op.attn_contiguous_ref(q[L - 1:L], K, V, [L - 1], pr.scale)[0])


def pin_causality():
    """Changing K/V at positions after p leaves query row p bit-identical."""
    pr = Problem(seed=10, lens=(13,))
    q, K, V = pr.dense(0)
    p = 6
    K2, V2 = K.copy(), V.copy()
    K2[p + 1:] += 5.0
    V2[p + 1:] -= 3.0
    a = op.attn_contiguous_ref(q[:p + 1], K, V, np.arange(p + 1), pr.scale)
    b = op.attn_contiguous_ref(q[:p + 1], K2, V2, np.arange(p + 1), pr.scale)
    assert np.array_equal(a, b)
    full = _rows(pr.prefill([0]), pr.lens, [0])[0]
    assert not np.array_equal(full[p + 1], op.attn_contiguous_ref(q[p + 1:p + 2], K2, V2, [p + 1], pr.scale)[0])


def pin_decode_equals_last_prefill_row():
    """Decode at len - 1 equals the last row of an uncached prefill."""
    pr = Problem(seed=11, lens=(5, 12, 8))
    d = pr.decode()
    rows = _rows(pr.prefill([0, 0, 0]), pr.lens, [0, 0, 0])
    for b in range(len(pr.lens)):
        np.testing.assert_allclose(d[b], rows[b][-1], rtol=1e-12, atol=1e-14)


def pin_chunked_equals_oneshot():
    """Prefill from num_cached = c (prefix hit or chunk continuation) equals
    the last rows of the one-shot prefill, for every c."""
    pr = Problem(seed=12, lens=(11, 7))
    full = _rows(pr.prefill([0, 0]), pr.lens, [0, 0])
    for c0 in range(pr.lens[0]):
        for c1 in (0, 3, 6):
            rows = _rows(pr.prefill([c0, c1]), pr.lens, [c0, c1])
            np.testing.assert_allclose(rows[0], full[0][c0:], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(rows[1], full[1][c1:], rtol=1e-12, atol=1e-14)


def _tagged_v(rng, lens, H, D):
    K = [_bf16_bits(rng.standard_normal((L, H, D))) for L in lens]
    V = []
    for L in lens:
        v = np.zeros((L, H, D))
        for g in range(H):
            v[:, g, :] = g + 1
        V.append(_bf16_bits(v))
    return K, V


def pin_head_tag():
    """V of KV head g is the constant g + 1: query head h must return
    h // (H_q / H_kv) + 1 (consecutive query heads share a KV head)."""
    pr = Problem(seed=13, Hq=8, Hkv=2, lens=(6, 10), kv=_tagged_v)
    G = pr.Hq // pr.Hkv
    out = pr.decode()
    for h in range(pr.Hq):
        np.testing.assert_allclose(out[:, h], h // G + 1, rtol=1e-12)


def pin_brute_force():
    """The vectorised oracle equals a scalar brute force on tiny inputs, for
    every cached-prefix length."""
    pr = Problem(seed=14, B=4, D=8, Hq=4, Hkv=2, lens=(13, 5))
    for cached in ([0, 0], [5, 4], [12, 1], [4, 2]):
        out = pr.prefill(cached)
        q_bits, q_pos, seq_of = [], [], []
        for b, c in enumerate(cached):
            for i in range(c, pr.lens[b]):
                q_bits.append(pr.qsrc[b][i].tolist())
                q_pos.append(i)
                seq_of.append(b)
        ref = np.asarray(brute_paged_attention(q_bits, q_pos, seq_of, pr.kc.tolist(), pr.vc.tolist(),
                                               pr.tables, pr.B, pr.Hq, pr.Hkv, pr.D, pr.scale))
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)


def pin_sdpa():
    """Equals torch's fp64 CPU scaled_dot_product_attention (an independent
    library implementation) with a bottom-right causal boolean mask and K/V
    repeated per query-head group."""
    pr = Problem(seed=15, B=4, D=16, Hq=6, Hkv=3, lens=(17, 9, 12))
    cached = [5, 0, 11]
    rows = _rows(pr.prefill(cached), pr.lens, cached)
    G = pr.Hq // pr.Hkv
    for b, c in enumerate(cached):
        q, K, V = pr.dense(b)
        L = pr.lens[b]
        n = L - c
        qt = torch.from_numpy(q[c:]).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)
        vt = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)
        mask = torch.from_numpy(np.arange(L)[None, :] <= (c + np.arange(n))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=pr.scale)
        ref = ref.squeeze(0).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(rows[b], ref, rtol=1e-11, atol=1e-13)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _wrap_attn(transform):
    orig = op.attn_contiguous_ref

    def f(q, K, V, q_pos, scale):
        return orig(*transform(q, K, V, q_pos, scale))
    return f


MUTANTS = {
    "gqa_modulo": ("_kv_head_of", lambda h, group: h % 2 if group > 1 else h),
    "mask_excludes_self": ("_visible", lambda q_pos, L: np.arange(L)[None, :] < np.asarray(q_pos)[:, None]),
    "mask_top_left": ("_visible", lambda q_pos, L: np.arange(L)[None, :]
                      <= (np.asarray(q_pos) - np.asarray(q_pos)[0])[:, None]),
    "mask_none": ("_visible", lambda q_pos, L: np.ones((len(q_pos), L), dtype=bool)),
    "gather_swapped": ("_logical_to_physical", lambda row, L, B: np.asarray(row, np.int64)[
        np.minimum(np.arange(L) % B, len(row) - 1)] * B + np.arange(L) // B),
    "gather_no_table": ("_logical_to_physical", lambda row, L, B: np.arange(L, dtype=np.int64)),
    "slot_offset_off_by_one": ("_physical_slot", lambda t, pos, B: int(t[pos // B]) * B + (pos + 1) % B),
    "slot_block_by_offset": ("_physical_slot", lambda t, pos, B: int(t[min(pos % B, len(t) - 1)]) * B + pos // B),
    "no_scale": ("attn_contiguous_ref", "noscale"),
    "k_v_swapped": ("attn_contiguous_ref", "swap"),
    "q_pos_shift": ("attn_contiguous_ref", "shift"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    attr, repl = MUTANTS[name]
    if repl == "noscale":
        repl = _wrap_attn(lambda q, K, V, p, s: (q, K, V, p, 1.0))
    elif repl == "swap":
        repl = _wrap_attn(lambda q, K, V, p, s: (q, V, K, p, s))
    elif repl == "shift":
        repl = _wrap_attn(lambda q, K, V, p, s: (q, K, V, np.maximum(np.asarray(p) - 1, 0), s))
    monkeypatch.setattr(op, attr, repl)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"
