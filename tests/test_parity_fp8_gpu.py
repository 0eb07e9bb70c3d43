"""GPU parity of the FP8 (E4M3) KV cache against the CPU oracle (C ABI).

The write is compared bit for bit on whole pools: random rows, quotients a
few ulps either side of every rounding midpoint, saturating magnitudes, NaN,
skipped slots, and every bf16 bit pattern at seven scales (two outside the
range where the quantiser uses its split division).  Decode reads a pool the GPU wrote itself and is compared with
the oracle's attention over the pool the oracle wrote (the two pools are
first checked identical): single pass, split with the window-aware merge,
sliding window, four group / block-size shapes, and the FP8 Llama-3-8B decode
workload at full size (whole pools bit-exact, decode on sampled sequences).
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def scale_dev(x):
    return torch.tensor([x], dtype=torch.float32, device="cuda")


def write_fp8_gpu(case):
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ks, vs = scale_dev(case.k_scale), scale_dev(case.v_scale)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping),
                       k_scale=ks, v_scale=vs)
    return kc, vc, ks, vs


def write_fp8_oracle(case):
    return oracle.kv_write_fp8(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                               case.spec.block_size, case.spec.dtype, case.k_scale, case.v_scale)


# ---------------------------------------------------------------------------
# the write
# ---------------------------------------------------------------------------
def _hard_rows(rng, T, H, d, scale):
    """fp32 rows mixing N(0,1) draws, quotients within 3 ulps of every E4M3
    rounding midpoint (times the scale), saturating values, and NaN."""
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = np.float32((vals + np.append(vals[1:], 480.0)) / 2 * scale)
    near = [mids]
    for _ in range(3):
        near.append(np.nextafter(near[-1], np.float32(np.inf)))
    m = mids
    for _ in range(3):
        m = np.nextafter(m, np.float32(0))
        near.append(m)
    special = np.float32([448 * scale, 500 * scale, 1e30, np.inf, -np.inf, np.nan, 0.0, -0.0])
    pool = np.concatenate(near + [-x for x in near] + [special])
    x = rng.normal(0, 1, (T, H, d)).astype(np.float32)
    flat = x.reshape(-1)
    idx = rng.choice(flat.size, size=min(flat.size // 2, pool.size * 4), replace=False)
    flat[idx] = rng.choice(pool, size=idx.size)
    return x


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_kv_write_fp8_bit_exact(dtype):
    rng = np.random.default_rng(41)
    NB, H, bs, d, T = 40, 4, 16, 128, 300
    ks, vs = np.float32(6 / 448), np.float32(0.37)
    k = _hard_rows(rng, T, H, d, ks)
    v = _hard_rows(rng, T, H, d, vs)
    if dtype == wl.BF16:
        k, v = wl.f32_to_bf16_bits(np.nan_to_num(k, nan=0.0)), wl.f32_to_bf16_bits(np.nan_to_num(v, nan=0.0))
        k[0, 0, :4] = wl.BF16_NAN            # NaN rows through the bf16 path too
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    slots[::17] = -1
    kc = np.full((NB, H, bs, d), 0x7F, np.uint8)
    vc = kc.copy()
    okc, ovc = oracle.kv_write_fp8(kc, vc, k, v, slots, bs, dtype, ks, vs)
    dkc, dvc = to_dev(kc), to_dev(vc)
    ops.paged_kv_write(to_dev(k), to_dev(v), dkc, dvc, to_dev(slots), k_scale=scale_dev(ks), v_scale=scale_dev(vs))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dkc.cpu().numpy(), okc)
    np.testing.assert_array_equal(dvc.cpu().numpy(), ovc)


@pytest.mark.parametrize("scale", [6 / 448, 0.37, 1.0, 3e-3, 1e4, 1e-12, 1e12])
def test_kv_write_fp8_every_bf16_value(scale):
    # every bf16 bit pattern (NaNs, infinities, subnormals, both zeros) as K and
    # as V, in 512 tokens of one 128-dim head: whole pools bit-exact
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(512, 1, 128)
    k, v = bits, bits[::-1].copy()
    slots = np.random.default_rng(43).permutation(512).astype(np.int32)
    kc = np.zeros((32, 1, 16, 128), np.uint8)
    vc = kc.copy()
    sc = np.float32(scale)
    with np.errstate(invalid="ignore", over="ignore"):   # NaN and infinite inputs are part of the sweep
        okc, ovc = oracle.kv_write_fp8(kc, vc, k, v, slots, 16, wl.BF16, sc, sc)
    dkc, dvc = to_dev(kc), to_dev(vc)
    ops.paged_kv_write(to_dev(k), to_dev(v), dkc, dvc, to_dev(slots), k_scale=scale_dev(sc), v_scale=scale_dev(sc))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dkc.cpu().numpy(), okc)
    np.testing.assert_array_equal(dvc.cpu().numpy(), ovc)


def test_kv_write_fp8_into_float8_dtype_pool():
    # a torch float8_e4m3fn pool is the same bytes
    rng = np.random.default_rng(42)
    k = rng.normal(0, 1, (5, 2, 64)).astype(np.float32)
    slots = np.array([3, 0, 9, -1, 4], np.int32)
    kc = torch.full((2, 2, 8, 64), 0x7F, dtype=torch.uint8, device="cuda")
    kc8 = kc.clone().view(torch.float8_e4m3fn)
    vc8 = kc.clone().view(torch.float8_e4m3fn)
    ks = scale_dev(0.05)
    ops.paged_kv_write(to_dev(k), to_dev(k), kc8, vc8, to_dev(slots), k_scale=ks, v_scale=ks)
    okc, _ = oracle.kv_write_fp8(kc.cpu().numpy(), kc.cpu().numpy(), k, k, slots, 8, wl.F32, 0.05, 0.05)
    np.testing.assert_array_equal(kc8.view(torch.uint8).cpu().numpy(), okc)


# ---------------------------------------------------------------------------
# decode over an FP8 pool
# ---------------------------------------------------------------------------
SHAPES = {
    "g4_bs16": dict(batch=6, ctx_min=1, ctx_max=600, max_blocks_per_seq=38),
    "g8_bs32": dict(batch=5, num_q_heads=16, num_kv_heads=2, block_size=32, ctx_min=1, ctx_max=700,
                    max_blocks_per_seq=22),
    "g1_bs64": dict(batch=4, num_q_heads=4, num_kv_heads=4, block_size=64, ctx_min=1, ctx_max=500,
                    max_blocks_per_seq=8),
    "g2_bs16": dict(batch=7, num_q_heads=8, num_kv_heads=4, ctx_min=60, ctx_max=1000, max_blocks_per_seq=63),
}


def decode_fp8_gpu(case, kc, vc, ks, vs, ps, window):
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    if ps:
        B, Hq, d = case.q.shape
        P = ops.num_partitions(case.max_context_len, ps)
        po = torch.full((B, Hq, P, d), float("nan"), dtype=torch.float32, device="cuda")
        pl = torch.full((B, Hq, P), float("nan"), dtype=torch.float32, device="cuda")
        ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, part_out=po,
                                   part_lse=pl, window=window, k_scale=ks, v_scale=vs)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, window=window)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale,
                                              window=window, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return to_host_f64(out), to_host_f64(lse)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_fp8_matches_oracle(name):
    case = wl.make_case(8, **SHAPES[name])
    bs = case.spec.block_size
    kc, vc, ks, vs = write_fp8_gpu(case)
    okc, ovc = write_fp8_oracle(case)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
    for window in (0, 100):
        ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, case.scale,
                                         case.spec.dtype, window=window, kv_dtype=oracle.E4M3,
                                         k_scale=case.k_scale, v_scale=case.v_scale)
        for ps in (0, bs * 4):
            out, lse = decode_fp8_gpu(case, kc, vc, ks, vs, ps, window)
            assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"{name} ps={ps} window={window}")


@pytest.mark.parametrize("name", ["g4_bs16", "g2_bs16"])
def test_decode_fp8_growing_scores(name):
    # every row written at position p is slope * p along one direction u and
    # every query lies along u, so the scores grow along the positions (the
    # E4M3 codes keep them monotone): the running max and O are rescaled at
    # nearly every tile with the K scale folded into the softmax scale, and the
    # split partitions carry lse values far apart
    case = wl.make_case(8, **SHAPES[name])
    rng = np.random.default_rng(9)
    d = case.spec.head_dim
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    pos = np.concatenate([np.arange(int(c)) for c in case.context_lens]).astype(np.float64)
    assert pos.size == case.k_new.shape[0]   # rows in (sequence, position) order
    k = 0.3 * pos[:, None, None] * u[None, None, :] + 0.01 * rng.standard_normal(case.k_new.shape)
    case.k_new = wl.f32_to_bf16_bits(k.astype(np.float32))
    case.q = wl.f32_to_bf16_bits((4.0 * u[None, None, :] + 0.01 * rng.standard_normal(case.q.shape))
                                 .astype(np.float32))
    case.k_scale = float(np.float32(0.5))   # keeps 0.3 * p * u inside the E4M3 range
    bs = case.spec.block_size
    kc, vc, ks, vs = write_fp8_gpu(case)
    okc, ovc = write_fp8_oracle(case)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, case.scale,
                                     case.spec.dtype, kv_dtype=oracle.E4M3, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    assert ref_lse.max() > 40.0
    for ps in (0, bs * 4):
        out, lse = decode_fp8_gpu(case, kc, vc, ks, vs, ps, 0)
        assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"growing {name} ps={ps}")


def test_decode_fp8_scales_are_read_from_device():
    # changing only the device scalars changes the result as the oracle says
    # (scales near the written ones keep outputs O(1), where the bf16 bar applies)
    case = wl.make_case(8, **SHAPES["g4_bs16"])
    kc, vc, _, _ = write_fp8_gpu(case)
    okc, ovc = write_fp8_oracle(case)
    for k_s, v_s in ((0.02, 0.016), (0.008, 0.009)):
        ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens,
                                         case.spec.block_size, case.scale, case.spec.dtype, kv_dtype=oracle.E4M3,
                                         k_scale=k_s, v_scale=v_s)
        out, lse = decode_fp8_gpu(case, kc, vc, scale_dev(k_s), scale_dev(v_s), 64, 0)
        assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"scales {k_s} {v_s}")


def test_decode_fp8_rejects_unsupported_shapes():
    case = wl.make_case(8, **SHAPES["g4_bs16"])
    kc, vc, ks, vs = write_fp8_gpu(case)
    q32 = to_dev(case.q).float()
    with pytest.raises(ops.PagedAttnError):
        ops.paged_attention_decode(q32, kc, vc, to_dev(case.block_tables), to_dev(case.context_lens),
                                   case.max_context_len, case.scale, k_scale=ks, v_scale=vs)
    with pytest.raises(ValueError):
        ops.paged_attention_decode(to_dev(case.q), kc, vc, to_dev(case.block_tables), to_dev(case.context_lens),
                                   case.max_context_len, case.scale)


# ---------------------------------------------------------------------------
# the FP8 decode workload at full size
# ---------------------------------------------------------------------------
def test_fp8_workload_full_size():
    case = wl.make_case(8)
    bs = case.spec.block_size
    kc, vc, ks, vs = write_fp8_gpu(case)
    okc, ovc = write_fp8_oracle(case)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
    ps = case.spec.partition_size
    out, lse = decode_fp8_gpu(case, kc, vc, ks, vs, ps, 0)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, case.scale,
                                     case.spec.dtype, kv_dtype=oracle.E4M3, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, "FP8 workload, every (sequence, head)")


def test_decode_fp8_long_tables():
    # more than 64 blocks per wave: the window of block ids is reloaded mid-unit
    case = wl.make_case(8, batch=3, ctx_fixed=(4200, 8193, 12000), max_blocks_per_seq=750)
    bs = case.spec.block_size
    kc, vc, ks, vs = write_fp8_gpu(case)
    okc, ovc = write_fp8_oracle(case)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, case.scale,
                                     case.spec.dtype, kv_dtype=oracle.E4M3, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    for ps in (0, 512, 4096):
        out, lse = decode_fp8_gpu(case, kc, vc, ks, vs, ps, 0)
        assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"long tables ps={ps}")
