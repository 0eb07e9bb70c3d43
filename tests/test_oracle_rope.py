"""Pins of the RoPE part of the oracle, CPU only.

The rotation is pinned by what the mathematics fixes, not by re-running its
own formula: position 0 is the identity; the half-split pairing is the
multiplication of z = x[:h] + i x[h:] by exp(i p theta) (numpy complex
arithmetic); each pair keeps its length; the score of a rotated query and key
depends on their positions only through the difference; the frequencies form
a geometric sequence starting at 1 with ratio base^(-2/rot_dim); dims past
rot_dim pass through.  The rounding to bf16 is pinned against torch's fp32 ->
bf16 cast (single rounding) and hand-worked ties, and the fused write against
the plain cache write of the rotated rows.  Planted mistakes at the end.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from oracle import attention as oa
from tests.test_oracle_pins import rand_f32

BASE = 10000.0


def test_position_zero_is_identity():
    x = rand_f32(np.random.default_rng(1), 5, 3, 64)
    np.testing.assert_array_equal(rope.rotate(x, np.zeros(5, np.int64), 64, BASE, oracle.F32), x.astype(np.float64))


@pytest.mark.parametrize("rot_dim,d", [(64, 64), (128, 128), (32, 64)])
def test_rotation_is_complex_multiplication(rot_dim, d):
    rng = np.random.default_rng(2)
    x = rand_f32(rng, 7, 2, d)
    pos = rng.integers(0, 20000, 7)
    y = rope.rotate(x, pos, rot_dim, BASE, oracle.F32)
    h = rot_dim // 2
    theta = BASE ** (-(np.arange(h) * 2.0) / rot_dim)
    z = x[..., :h].astype(np.float64) + 1j * x[..., h:rot_dim].astype(np.float64)
    zr = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    np.testing.assert_allclose(y[..., :h], zr.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(y[..., h:rot_dim], zr.imag, rtol=0, atol=1e-9)
    np.testing.assert_array_equal(y[..., rot_dim:], x[..., rot_dim:].astype(np.float64))   # pass-through dims
    # every pair keeps its length
    np.testing.assert_allclose(np.abs(y[..., :h] + 1j * y[..., h:rot_dim]), np.abs(z), rtol=1e-12, atol=0)


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(3)
    q = rand_f32(rng, 1, 1, 128)
    k = rand_f32(rng, 1, 1, 128)
    def score(p, s):
        return float((rope.rotate(q, [p], 128, BASE, oracle.F32) * rope.rotate(k, [s], 128, BASE, oracle.F32)).sum())
    for p, s, t in ((5, 2, 100), (1000, 17, 3000), (0, 0, 7)):
        assert abs(score(p, s) - score(p + t, s + t)) < 1e-9
    assert abs(score(5, 2) - score(2, 5)) > 1e-6   # but not on its sign


def test_frequencies():
    th = rope.inv_freq(128, BASE)
    assert th[0] == 1.0 and len(th) == 64
    np.testing.assert_allclose(th[1:] / th[:-1], np.full(63, BASE ** (-2.0 / 128)), rtol=1e-13)
    assert abs(th[-1] - 10.0 ** (-4 * 126 / 128)) < 1e-18
    tab = rope.cos_sin_table(8, 128, BASE)
    assert tab.shape == (8, 128)
    np.testing.assert_array_equal(tab[0], np.concatenate([np.ones(64), np.zeros(64)]))
    assert abs(tab[1, 0] - np.cos(1.0)) < 1e-15 and abs(tab[1, 64] - np.sin(1.0)) < 1e-15


def test_round_to_bf16():
    rng = np.random.default_rng(4)
    x32 = np.concatenate([rng.normal(0, 3, 50000), rng.normal(0, 1e-3, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(rope.round_to(x32.astype(np.float64), oracle.BF16), ref)
    # ties to even, and a value whose fp32 rounding would land on a tie
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -2.2734374098623973])
    np.testing.assert_array_equal(rope.round_to(x, oracle.BF16),
                                  np.array([0x3F80, 0x3F82, 0xBF80, 0x0000, 0xC011], np.uint16))


def test_fused_write_is_rotation_then_plain_write():
    rng = np.random.default_rng(5)
    T, Hq, Hkv, d, bs, NB = 6, 4, 2, 64, 8, 5
    q, k, v = rand_f32(rng, T, Hq, d), rand_f32(rng, T, Hkv, d), rand_f32(rng, T, Hkv, d)
    kc = np.full((NB, Hkv, bs, d), np.nan, np.float32)
    vc = kc.copy()
    slots = np.array([3, 9, -1, 17, 0, 30], np.int32)
    pos = np.array([0, 5, 9, 100, 4095, 7], np.int64)
    qr, kr, okc, ovc = rope.rope_kv_write(q, k, v, kc, vc, slots, pos, bs, d, BASE, oracle.F32)
    np.testing.assert_array_equal(qr, rope.rotate(q, pos, d, BASE, oracle.F32).astype(np.float32))
    for t, s in enumerate(slots):
        if s >= 0:
            np.testing.assert_array_equal(okc[s // bs, :, s % bs], kr[t])
            np.testing.assert_array_equal(ovc[s // bs, :, s % bs], v[t])   # v is not rotated
    assert np.isnan(okc[0, :, 1]).all()                                    # untouched slot


def test_decode_after_fused_write_is_shift_invariant():
    # attention of rotated rows depends on positions through differences only:
    # shifting every position of a sequence by t leaves decode unchanged
    rng = np.random.default_rng(6)
    n, Hq, Hkv, d, bs = 40, 4, 2, 64, 8
    q, k, v = rand_f32(rng, 1, Hq, d), rand_f32(rng, n, Hkv, d), rand_f32(rng, n, Hkv, d)
    tables = np.arange(5, dtype=np.int32)[None, :]
    slots = np.arange(n, dtype=np.int32)
    outs = []
    for t in (0, 1234):
        pos = np.arange(n) + t
        kc = np.zeros((5, Hkv, bs, d), np.float32)
        _, _, kc, vc = rope.rope_kv_write(np.zeros((n, Hq, d), np.float32), k, v, kc, kc.copy(), slots, pos, bs, d,
                                          BASE, oracle.F32)
        qr = rope.round_to(rope.rotate(q, [n - 1 + t], d, BASE, oracle.F32), oracle.F32)
        outs.append(oracle.decode(qr, kc, vc, tables, np.array([n], np.int32), bs, 0.125, oracle.F32))
    np.testing.assert_allclose(outs[0][0], outs[1][0], rtol=0, atol=2e-6)
    np.testing.assert_allclose(outs[0][1], outs[1][1], rtol=0, atol=2e-6)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def _rotate_interleaved(x, positions, rot_dim, base, dtype):
    x = oa.upcast(x, dtype).copy()
    ang = np.asarray(positions, np.float64)[:, None] * rope.inv_freq(rot_dim, base)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., 0:rot_dim:2].copy(), x[..., 1:rot_dim:2].copy()
    x[..., 0:rot_dim:2], x[..., 1:rot_dim:2] = a * c - b * s, b * c + a * s
    return x


def _rotate_backwards(x, positions, rot_dim, base, dtype):
    return rope.__dict__["_orig_rotate"](x, -np.asarray(positions), rot_dim, base, dtype)


def _rotate_shifted(x, positions, rot_dim, base, dtype):
    return rope.__dict__["_orig_rotate"](x, np.asarray(positions) + 1, rot_dim, base, dtype)


def _inv_freq_half(rot_dim, base):
    return np.power(float(base), -np.arange(rot_dim // 2, dtype=np.float64) / rot_dim)


def _round_ties_away(x64, dtype):
    f = np.asarray(x64, np.float64)
    if dtype == oracle.F32:
        return f.astype(np.float32)
    _, E = np.frexp(f)
    step = np.ldexp(1.0, E - 8)
    r = np.sign(f) * np.floor(np.abs(f) / step + 0.5) * step
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


ROPE_MUTANTS = {
    "pairs_interleaved": [("rotate", _rotate_interleaved)],
    "rotates_backwards": [("rotate", _rotate_backwards)],
    "position_off_by_one": [("rotate", _rotate_shifted)],
    "frequency_exponent_halved": [("inv_freq", _inv_freq_half)],
    "rounding_ties_away": [("round_to", _round_ties_away)],
}

ROPE_PINS = [
    test_position_zero_is_identity,
    lambda: test_rotation_is_complex_multiplication(64, 64),
    test_frequencies,
    test_round_to_bf16,
]


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setitem(rope.__dict__, "_orig_rotate", rope.rotate)
    for attr, repl in ROPE_MUTANTS[name]:
        monkeypatch.setattr(rope, attr, repl)
    caught = 0
    for pin in ROPE_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught mutant {name}"
