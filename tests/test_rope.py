"""Rotary embedding fused with the KV store: the oracle's pins (mathematics, no
GPU), the host cos/sin table against the oracle's angles, and argument
validation of rope_kv_store."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_attention_28_amd as P
from oracle import paged as op
from oracle import rope as orope


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_position_zero_is_identity():
    x = _rand((5, 3, 128), 1)
    np.testing.assert_array_equal(orope.rope_ref(x, np.zeros(5)), x)


def test_pairs_keep_their_norm():
    x = _rand((7, 2, 128), 2)
    y = orope.rope_ref(x, np.arange(7) * 1000 + 3)
    nx = x[..., :64] ** 2 + x[..., 64:] ** 2
    ny = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12)


def test_rotations_compose():
    x = _rand((6, 2, 128), 3)
    a = np.array([0, 1, 5, 100, 4000, 30000])
    b = np.array([7, 0, 9, 2, 123, 9000])
    two = orope.rope_ref(orope.rope_ref(x, a), b)
    np.testing.assert_allclose(two, orope.rope_ref(x, a + b), rtol=1e-9, atol=1e-9)


def test_scores_depend_on_relative_position_only():
    q = _rand((1, 4, 128), 4)
    k = _rand((1, 4, 128), 5)
    for p, r in ((10, 3), (500, 499), (20000, 1)):
        base = np.einsum("nhd,nhd->h", orope.rope_ref(q, [p]), orope.rope_ref(k, [r]))
        for shift in (1, 77, 4096):
            moved = np.einsum("nhd,nhd->h", orope.rope_ref(q, [p + shift]), orope.rope_ref(k, [r + shift]))
            np.testing.assert_allclose(moved, base, rtol=1e-9, atol=1e-9)


def test_every_head_turns_the_same_way():
    one = _rand((3, 1, 128), 9)
    x = np.repeat(one, 6, axis=1)                 # six identical heads
    y = orope.rope_ref(x, [1, 40, 7000])
    for h in range(1, 6):
        np.testing.assert_array_equal(y[:, h], y[:, 0])
    assert np.abs(y - x).max() > 1e-3             # and they did turn


def test_two_dims_are_the_plane_rotation():
    x = _rand((4, 1, 2), 6)
    pos = np.array([0.0, 1.0, 2.5, 31.0])
    y = orope.rope_ref(x, pos, theta=123.0)   # one pair, frequency theta^0 = 1
    c, s = np.cos(pos), np.sin(pos)
    np.testing.assert_allclose(y[:, 0, 0], c * x[:, 0, 0] - s * x[:, 0, 1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[:, 0, 1], s * x[:, 0, 0] + c * x[:, 0, 1], rtol=1e-14, atol=1e-15)


GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "rope_angles_closed_form.json")


def test_unit_vectors_turn_by_the_hand_worked_angles():
    """Pins the frequency schedule: unit vectors along dim i rotate to (cos a_i, sin a_i) on dims (i, i + D/2),
    with the angles a_i worked out by hand for theta = 10^4, D = 8 (pair i turns at 10^-i rad per position)
    and for theta = 10^6, D = 128 (pairs 0 and 32), in tests/golden/rope_angles_closed_form.json."""
    import json
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        D = c["head_dim"]
        pairs = c.get("pairs", list(range(D // 2)))
        for i, a in zip(pairs, c["angles"]):
            x = np.zeros((1, 1, D))
            x[0, 0, i] = 1.0
            y = orope.rope_ref(x, [c["pos"]], theta=c["theta"])[0, 0]
            want = np.zeros(D)
            want[i], want[i + D // 2] = np.cos(a), np.sin(a)
            np.testing.assert_allclose(y, want, rtol=0, atol=1e-9, err_msg=f"D={D} pos={c['pos']} pair {i}")


def test_bf16_rounding_matches_torch():
    x = np.concatenate([_rand(10000, 7) * 10, [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.3e-39]])
    bits = orope.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_fused_store_reference():
    rng = np.random.default_rng(8)
    n, hq, hkv = 9, 4, 2
    q = orope.f64_to_bf16_bits(rng.standard_normal((n, hq, 128)))
    k = orope.f64_to_bf16_bits(rng.standard_normal((n, hkv, 128)))
    v = orope.f64_to_bf16_bits(rng.standard_normal((n, hkv, 128)))
    pos = rng.integers(0, 5000, size=n)
    slots = np.array([3, -1, 0, 7, 12, -1, 15, 4, 9], dtype=np.int32)
    kc = np.full((4, 4, hkv, 128), 0x7FC0, dtype=np.uint16)
    vc = kc.copy()
    q_rot, k_rot, kc2, vc2 = orope.rope_kv_store_ref(q, k, v, pos, slots, kc, vc)
    flat_k, flat_v = kc2.reshape(16, hkv, 128), vc2.reshape(16, hkv, 128)
    for t, sl in enumerate(slots):
        if sl >= 0:
            np.testing.assert_array_equal(flat_v[sl], v[t])                       # V: bit copy
            np.testing.assert_array_equal(flat_k[sl], orope.f64_to_bf16_bits(k_rot[t]))
    untouched = np.setdiff1d(np.arange(16), slots[slots >= 0])
    assert (flat_k[untouched] == 0x7FC0).all() and (flat_v[untouched] == 0x7FC0).all()
    np.testing.assert_allclose(q_rot, orope.rope_ref(q, pos))


@pytest.mark.parametrize("mutant", ["k_turns_backwards", "one_head_unrotated", "exponent_i_over_d",
                                    "pairs_interleaved"])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    real = orope.rope_ref
    real_angles = orope.rope_angles
    if mutant == "exponent_i_over_d":          # theta^(-i/D) instead of theta^(-2i/D)
        def angles(positions, head_dim, theta=orope.DEFAULT_THETA):
            i = np.arange(head_dim // 2, dtype=np.float64)
            return np.asarray(positions, dtype=np.float64)[:, None] * (theta ** (-i / head_dim))[None, :]
        monkeypatch.setattr(orope, "rope_angles", angles)
    if mutant == "pairs_interleaved":          # pair (2i, 2i + 1) instead of (i, i + D/2)
        def inter(x, positions, theta=orope.DEFAULT_THETA):
            x = op.bf16_bits_to_f64(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
            D = x.shape[-1]
            a = real_angles(positions, D, theta)[:, None, :]
            c, s = np.cos(a), np.sin(a)
            y = x.copy()
            y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
            y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
            return y
        monkeypatch.setattr(orope, "rope_ref", inter)

    def bad(x, positions, theta=orope.DEFAULT_THETA, _k=[0]):
        y = real(x, positions, theta)
        _k[0] += 1
        if mutant == "k_turns_backwards" and _k[0] % 2 == 0:
            return real(x, -np.asarray(positions, dtype=np.float64), theta)
        if mutant == "one_head_unrotated" and y.shape[1] > 1:
            y = y.copy()
            y[:, 1] = op.bf16_bits_to_f64(x)[:, 1] if np.asarray(x).dtype == np.uint16 else np.asarray(x)[:, 1]
        return y

    if mutant in ("k_turns_backwards", "one_head_unrotated"):
        monkeypatch.setattr(orope, "rope_ref", bad)
    failed = 0
    for pin in (test_position_zero_is_identity, test_pairs_keep_their_norm, test_rotations_compose,
                test_scores_depend_on_relative_position_only, test_every_head_turns_the_same_way,
                test_unit_vectors_turn_by_the_hand_worked_angles):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, mutant


def test_host_table_matches_oracle_angles():
    tab = P.pkv_rope_cos_sin(4096, 128, 1.0e6)
    a = orope.rope_angles(np.arange(4096), 128, 1.0e6)
    np.testing.assert_allclose(tab[:, :64], np.cos(a), rtol=0, atol=6e-8)
    np.testing.assert_allclose(tab[:, 64:], np.sin(a), rtol=0, atol=6e-8)
    with pytest.raises(P.PkvError):
        P.pkv_rope_cos_sin(10, 127)


F = 0x10000  # a fake, 16-byte aligned "device" pointer: never dereferenced on these paths


def test_rope_kv_store_validation():
    lib = P.load_library()
    args = lambda **kw: [kw.get("q", F), kw.get("qs", 2048), F, kw.get("ks", 1024), F, 1024, F, kw.get("tab", F),
                         kw.get("maxpos", 4096), F, F, F, kw.get("T", 100), kw.get("hq", 16), kw.get("hkv", 8),
                         kw.get("d", 128), 256, 100, None]
    assert lib.rope_kv_store(*args(d=64)) == 2
    assert lib.rope_kv_store(*args(hkv=3)) == 2
    assert lib.rope_kv_store(*args(hq=65)) == 2
    assert lib.rope_kv_store(*args(qs=1024)) == 1          # stride smaller than a 16-head row
    assert lib.rope_kv_store(*args(ks=1028)) == 2          # stride not a multiple of 8
    assert lib.rope_kv_store(*args(q=None)) == 1
    assert lib.rope_kv_store(*args(tab=F + 4)) == 2        # table misaligned
    assert lib.rope_kv_store(*args(maxpos=0)) == 1
    assert lib.rope_kv_store(*args(T=0)) == 0
