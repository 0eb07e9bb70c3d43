"""Pins of the FP8 (E4M3) part of the oracle, CPU only.

The encoding is pinned to what does not come from the oracle itself:
  * the fixed values of the OCP 8-bit floating point specification's E4M3
    format (bias 7, max 448, smallest normal 2^-6, smallest subnormal 2^-9,
    S.1111.111 NaN, no infinities);
  * torch's own float8_e4m3fn decode of all 256 codes and its round-to-
    nearest-even cast of in-range fp32 values (an independent implementation;
    torch does not saturate, so the saturation is pinned by closed forms);
  * attention over an FP8 cache equals torch float64 SDPA over K and V that
    torch dequantised (its float8 decode times the scale).
A mutant harness at the end plants plausible mistakes in the FP8 oracle and
checks that these pins catch each.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3 as e4m3_mod
from oracle import fp8 as fp8_mod
from oracle import attention as oa
from tests.test_oracle_pins import paged_batch, page_window_mask, rand_f32


def torch_decode_codes(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# the code table
# ---------------------------------------------------------------------------
def test_e4m3_values_match_the_format_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_value(codes)
    ref = torch_decode_codes(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    # fixed points of the E4M3 definition
    v = lambda c: float(oracle.e4m3_value(np.array([c], np.uint8))[0])
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6 and v(0x07) == 7 * 2.0 ** -9 and v(0x01) == 2.0 ** -9
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x30) == 0.5
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert np.isnan(mine).sum() == 2   # no other NaN and no infinity
    assert np.all(np.diff(mine[:0x7F]) > 0)


def _sweep():
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    nxt = np.append(vals[1:], 480.0)
    mids = (vals + nxt) / 2
    xs = [vals, mids]
    m32 = mids.astype(np.float32)
    xs += [np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    rng = np.random.default_rng(7)
    for sigma in (1e-3, 0.05, 1.0, 30.0):
        xs.append(rng.normal(0, sigma, 4000))
    x = np.concatenate([np.asarray(a, np.float64) for a in xs]).astype(np.float32)
    x = x[np.abs(x) < 464]          # torch does not saturate past the last midpoint
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch_in_range():
    x = _sweep()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), torch_encode(x))


def test_e4m3_encode_saturates_and_keeps_nan():
    x = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e30, np.inf], np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(x), np.full(7, 0x7E, np.uint8))
    np.testing.assert_array_equal(oracle.e4m3_encode(-x), np.full(7, 0xFE, np.uint8))
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_value(codes).astype(np.float32)), codes)
    # exact halfway points go to the even code: 2^-10 -> 0, 1.0625 -> 1.0 (0x38), 1.1875 -> 1.25 (0x3A)
    x = np.array([2.0 ** -10, 1.0625, 1.1875, 3 * 2.0 ** -10], np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(x), np.array([0x00, 0x38, 0x3A, 0x02], np.uint8))


# ---------------------------------------------------------------------------
# quantised write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_quantize_is_fp32_division_then_nearest(dtype):
    rng = np.random.default_rng(3)
    scale = np.float32(6.0 / 448.0)
    # random rows, plus inputs whose quotient lands within a few ulps of a
    # rounding midpoint (where the exact fp32 division decides the code)
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals + np.append(vals[1:], 480.0)) / 2
    near = np.float32(mids * float(scale))
    steps = [near]
    for k in range(1, 4):
        steps += [np.nextafter(steps[-1], np.float32(np.inf))]
    down = [near]
    for k in range(1, 4):
        down += [np.nextafter(down[-1], np.float32(0))]
    x32 = np.concatenate([rng.normal(0, 2, 20000).astype(np.float32)] + steps + down[1:])
    if dtype == oracle.BF16:
        from attention_paged_kv_write_amd.workloads import f32_to_bf16_bits
        x = f32_to_bf16_bits(x32)
        xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    else:
        x = x32
        xf = torch.from_numpy(x32)
    q = (xf / torch.tensor(scale)).numpy()
    keep = np.abs(q) < 464
    np.testing.assert_array_equal(oracle.quantize(x, dtype, scale)[keep], torch_encode(q[keep]))
    assert np.all(oracle.quantize(x, dtype, scale)[~keep] & 0x7F == 0x7E)


def test_kv_write_fp8_scatters_codes():
    rng = np.random.default_rng(4)
    NB, Hkv, bs, d, T = 6, 2, 4, 16, 9
    k = rand_f32(rng, T, Hkv, d)
    v = rand_f32(rng, T, Hkv, d) * 3
    kc = np.full((NB, Hkv, bs, d), 0x7F, np.uint8)
    vc = kc.copy()
    slots = np.array([0, 5, 23, -1, 7, 12, 1, 22, 3], np.int32)
    ks, vs = np.float32(0.02), np.float32(0.01)
    okc, ovc = oracle.kv_write_fp8(kc, vc, k, v, slots, bs, oracle.F32, ks, vs)
    rk = kc.copy()
    rv = vc.copy()
    tk = torch_encode(torch.from_numpy(k).div(torch.tensor(ks)).numpy().clip(-448, 448))
    tv = torch_encode(torch.from_numpy(v).div(torch.tensor(vs)).numpy().clip(-448, 448))
    for t, s in enumerate(slots):
        if s >= 0:
            rk[s // bs, :, s % bs, :] = tk[t]
            rv[s // bs, :, s % bs, :] = tv[t]
    np.testing.assert_array_equal(okc, rk)
    np.testing.assert_array_equal(ovc, rv)
    assert (okc[0, :, 2, :] == 0x7F).all()   # untouched slot keeps its code


# ---------------------------------------------------------------------------
# attention over an FP8 cache
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("window", [0, 9])
def test_fp8_decode_equals_sdpa_on_torch_dequantised_kv(window):
    rng = np.random.default_rng(5)
    Hq, Hkv, d, bs, lens = 4, 2, 16, 8, (1, 9, 30, 57)
    ks, vs = np.float32(4.5 / 448.0), np.float32(5.0 / 448.0)
    Ks = [rand_f32(rng, n, Hkv, d) for n in lens]
    Vs = [rand_f32(rng, n, Hkv, d) for n in lens]
    assert max(np.abs(x).max() for x in Ks) < 4.4 and max(np.abs(x).max() for x in Vs) < 4.9   # codes in range
    # codes of every row (torch's cast; in range by the scales' choice)
    Kc = [torch_encode((torch.from_numpy(K) / torch.tensor(ks)).numpy()) for K in Ks]
    Vc = [torch_encode((torch.from_numpy(V) / torch.tensor(vs)).numpy()) for V in Vs]
    # page the codes (carried as float32; unused slots come back NaN -> the NaN code)
    kp, vp, tables, ctx = paged_batch([c.astype(np.float32) for c in Kc], [c.astype(np.float32) for c in Vc],
                                      bs, rng)
    kp = np.where(np.isnan(kp), 0x7F, kp).astype(np.uint8)
    vp = np.where(np.isnan(vp), 0x7F, vp).astype(np.uint8)
    q = rand_f32(rng, len(lens), Hq, d)
    out, lse = oracle.decode(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, window=window,
                             kv_dtype=oracle.E4M3, k_scale=ks, v_scale=vs)
    for b, n in enumerate(lens):
        K = torch.from_numpy(torch_decode_codes(Kc[b]) * float(ks)).permute(1, 0, 2).repeat_interleave(2, 0)
        V = torch.from_numpy(torch_decode_codes(Vc[b]) * float(vs)).permute(1, 0, 2).repeat_interleave(2, 0)
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        allowed = page_window_mask(1, n, window, offset=n - 1) if window else torch.ones((1, n), dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=allowed,
                                                                scale=0.25)[0, :, 0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)
        S = ((Q @ K.transpose(1, 2)) * 0.25).masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(lse[b], torch.logsumexp(S, -1)[:, 0].numpy(), rtol=0, atol=1e-12)
    po, pl = oracle.decode_partitions(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, 16, window=window,
                                      kv_dtype=oracle.E4M3, k_scale=ks, v_scale=vs)
    mo, ml = oracle.reduce_partitions(po, pl, ctx, 16, window=window)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def _encode_ties_away(x):
    x = np.asarray(x, np.float32)
    a = np.abs(x.astype(np.float64))
    T = e4m3_mod._POS_VALUES
    hi = np.clip(np.searchsorted(T, np.minimum(a, 448.0)), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where(T[hi] - a <= a - T[lo], hi, lo)
    code = np.where(a >= 448.0, 0x7E, code)
    out = np.where(np.signbit(x), 0x80, 0) | code
    return np.where(np.isnan(x), 0x7F, out).astype(np.uint8)


def _encode_no_saturation(x):
    x = np.asarray(x, np.float32)
    out = e4m3_mod.__dict__["_orig_encode"](x)
    return np.where(np.abs(x) >= 464, 0x7F | (out & 0x80), out).astype(np.uint8)


def _value_bias_8(codes):
    return e4m3_mod.__dict__["_orig_value"](codes) / 2.0


def _quantize_by_reciprocal(x, dtype, scale):
    q = oa.upcast(x, dtype).astype(np.float32) * (np.float32(1.0) / np.float32(scale))
    return fp8_mod.e4m3_encode(q)


def _kv_rows_no_scale(rows, dtype, kv_dtype, scale):
    return oa.upcast(rows, kv_dtype or dtype)


def _kv_rows_exponent_only(rows, dtype, kv_dtype, scale):
    # the scale's power of two only (what a hardware exponent-scaled convert does)
    if kv_dtype is None:
        return oa.upcast(rows, dtype)
    return oa.upcast(rows, kv_dtype) * 2.0 ** math.floor(math.log2(float(scale)))


FP8_MUTANTS = {
    "encode_ties_away_from_zero": [(e4m3_mod, "e4m3_encode", _encode_ties_away),
                                   (fp8_mod, "e4m3_encode", _encode_ties_away),
                                   (oracle, "e4m3_encode", _encode_ties_away)],
    "encode_overflow_to_nan": [(e4m3_mod, "e4m3_encode", _encode_no_saturation),
                               (fp8_mod, "e4m3_encode", _encode_no_saturation),
                               (oracle, "e4m3_encode", _encode_no_saturation)],
    "exponent_bias_8": [(e4m3_mod, "e4m3_value", _value_bias_8), (oa, "e4m3_value", _value_bias_8),
                        (oracle, "e4m3_value", _value_bias_8)],
    "quantize_by_reciprocal": [(fp8_mod, "quantize", _quantize_by_reciprocal),
                               (oracle, "quantize", _quantize_by_reciprocal)],
    "dequantize_ignores_scale": [(oa, "kv_rows", _kv_rows_no_scale)],
    "dequantize_exponent_only": [(oa, "kv_rows", _kv_rows_exponent_only)],
}

FP8_PINS = [
    test_e4m3_values_match_the_format_and_torch,
    test_e4m3_encode_matches_torch_in_range,
    test_e4m3_encode_saturates_and_keeps_nan,
    test_e4m3_round_trip_and_ties,
    lambda: test_quantize_is_fp32_division_then_nearest(oracle.F32),
    lambda: test_quantize_is_fp32_division_then_nearest(oracle.BF16),
    test_kv_write_fp8_scatters_codes,
    lambda: test_fp8_decode_equals_sdpa_on_torch_dequantised_kv(0),
]


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setitem(e4m3_mod.__dict__, "_orig_encode", e4m3_mod.e4m3_encode)
    monkeypatch.setitem(e4m3_mod.__dict__, "_orig_value", e4m3_mod.e4m3_value)
    for mod, attr, repl in FP8_MUTANTS[name]:
        monkeypatch.setattr(mod, attr, repl)
    caught = 0
    for pin in FP8_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught mutant {name}"
