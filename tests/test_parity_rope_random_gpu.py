"""Seeded random shapes for RoPE fused into the cache write (C ABI), against
the oracle's rotation and write.

Each case draws the dtype (bf16 / f32), head_dim (64 / 128), rot_dim (a
multiple of 16 up to head_dim), the base (LLaMA's 10000, 500000, or a
log-uniform draw over 100 .. 10^6), the GQA group and KV heads, the block
size, the sequence lengths, positions anywhere in tables of up to 131,072
rows, and slots with about one in ten set to -1.  The bar is the one the
fixed-shape RoPE tests derive: one unit in the last place of the result
(bf16) plus four fp32 ulps of |x1 c| + |x2 s|; the pool's k is bit-identical
to the k rotated in place, v is copied bit for bit, dims past rot_dim pass
through, and slots that are not written stay NaN.
"""
import numpy as np
import pytest
import torch

from oracle import rope
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import to_dev, to_host_bits
from tests.test_parity_rope_gpu import check_rotated

N_ROPE = 40


def rope_draw(i):
    rng = np.random.default_rng(7500 + i)
    dtype = wl.BF16 if rng.random() < 0.6 else wl.F32
    d = int(rng.choice([64, 128]))
    rot = 16 * int(rng.integers(1, d // 16 + 1))
    r = rng.random()
    base = 10000.0 if r < 0.4 else (500000.0 if r < 0.6 else float(np.exp(rng.uniform(np.log(100), np.log(1e6)))))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 5))
    S = int(rng.integers(1, 5))
    lens = tuple(int(x) for x in rng.integers(1, 200, S))
    max_pos = int(rng.choice([sum(lens) + 1, 4096, 131072]))
    return dict(seed=9500 + i, dtype=dtype, head_dim=d, rot=rot, base=base, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                block_size=int(rng.choice([8, 16, 32, 64])), num_seqs=S, lens_fixed=lens, max_pos=max_pos,
                pos_seed=int(rng.integers(1 << 30)))


def test_rope_draws_are_valid_and_cover_the_space():
    draws = [rope_draw(i) for i in range(N_ROPE)]
    for c in draws:
        assert c["rot"] % 16 == 0 and 16 <= c["rot"] <= c["head_dim"]
    assert {c["dtype"] for c in draws} == {wl.BF16, wl.F32}
    assert {c["head_dim"] for c in draws} == {64, 128}
    assert any(c["rot"] < c["head_dim"] for c in draws) and any(c["rot"] == c["head_dim"] for c in draws)
    assert {c["num_q_heads"] // c["num_kv_heads"] for c in draws} == {1, 2, 4, 8}
    assert {c["block_size"] for c in draws} == {8, 16, 32, 64}
    assert any(c["base"] == 10000.0 for c in draws) and any(c["base"] not in (10000.0, 500000.0) for c in draws)
    assert any(c["max_pos"] == 131072 for c in draws)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_ROPE), ids=lambda i: f"rope{i:02d}")
def test_random_rope_write(i):
    draw = rope_draw(i)
    print("rope", draw, flush=True)
    dtype, rot, base, bs = draw["dtype"], draw["rot"], draw["base"], draw["block_size"]
    case = wl.make_case(3, seed=draw["seed"], name="random_rope", dtype=dtype, head_dim=draw["head_dim"],
                        num_q_heads=draw["num_q_heads"], num_kv_heads=draw["num_kv_heads"], block_size=bs,
                        num_seqs=draw["num_seqs"], lens_fixed=draw["lens_fixed"])
    T, Hq, d = case.q.shape
    Hkv = case.k.shape[1]
    rng = np.random.default_rng(draw["pos_seed"])
    pos = rng.integers(0, draw["max_pos"], T).astype(np.int32)
    slots = case.slot_mapping.copy()
    slots[rng.random(T) < 0.1] = -1
    pool = wl.empty_pool(case.num_blocks, Hkv, bs, d, dtype)
    dq, dk, dv = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    kc, vc = to_dev(pool), to_dev(pool.copy())
    table = ops.rope_cos_sin_cache(draw["max_pos"], rot, base)
    ops.paged_kv_write_rope(dq, dk, dv, kc, vc, to_dev(slots), to_dev(pos), table)
    torch.cuda.synchronize()
    qr, kr, okc, ovc = rope.rope_kv_write(case.q, case.k, case.v, pool, pool.copy(), slots, pos, bs, rot, base,
                                          dtype)
    check_rotated(dq, qr, case.q, pos, rot, dtype, f"draw {i} q", base)
    check_rotated(dk, kr, case.k, pos, rot, dtype, f"draw {i} k", base)
    np.testing.assert_array_equal(to_host_bits(dq)[..., rot:], case.q[..., rot:])
    np.testing.assert_array_equal(to_host_bits(dk)[..., rot:], case.k[..., rot:])
    # the pool holds exactly the in-place k and the input v at written slots, NaN elsewhere
    gk, gv, k_inplace = to_host_bits(kc), to_host_bits(vc), to_host_bits(dk)
    want_k, want_v = pool.copy(), pool.copy()
    for t, s in enumerate(slots):
        if s >= 0:
            want_k[s // bs, :, s % bs] = k_inplace[t]
            want_v[s // bs, :, s % bs] = case.v[t]
    np.testing.assert_array_equal(gk, want_k)
    np.testing.assert_array_equal(gv, want_v)
    # and the oracle's write of its own rotation agrees wherever it is bit-exact
    assert np.array_equal(np.isnan(wl.bf16_bits_to_f32(okc) if dtype == wl.BF16 else okc),
                          np.isnan(wl.bf16_bits_to_f32(gk) if dtype == wl.BF16 else gk))
