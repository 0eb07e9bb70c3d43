"""GPU parity of RoPE fused into the cache write against the CPU oracle (C ABI).

The table is compared with the oracle's fp64 table rounded to fp32.  The fused
write rotates in fp32 (y = x1 c - x2 s) and rounds to the dtype once, the
oracle rounds the exact rotation once; the bar derived from that arithmetic is
one unit in the last place of the result (bf16) plus four fp32 ulps of
|x1 c| + |x2 s|, the error the fp32 products and difference can carry when
they cancel (f32 inputs: the fp32 term alone).  The pool's k is
bit-identical to the k rotated in place, v is copied bit for bit, dims past
rot_dim pass through unchanged, and negative slots write nothing.  A decode
over a cache written this way is compared with the oracle's chain.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

BASE = 10000.0


def bf16_ulp(ref64):
    _, E = np.frexp(np.abs(ref64))
    return np.ldexp(1.0, E - 8)


def positions_of(cu):
    cu = np.asarray(cu)
    return np.concatenate([np.arange(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]).astype(np.int32)


def test_cos_sin_table():
    for P, rot in ((4096, 128), (333, 64), (20000, 32)):
        tab = ops.rope_cos_sin_cache(P, rot, BASE).cpu().numpy()
        ref = rope.cos_sin_table(P, rot, BASE).astype(np.float32)
        np.testing.assert_allclose(tab, ref, rtol=0, atol=1.2e-7)
        assert (tab == ref).mean() > 0.999


def run_fused(case, dtype, rot, P=4096):
    T, Hq, d = case.q.shape
    Hkv = case.k.shape[1]
    pos = positions_of(case.cu_seqlens)
    NB, bs = case.num_blocks, case.spec.block_size
    pool = wl.empty_pool(NB, Hkv, bs, d, dtype)
    dq, dk, dv = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    kc, vc = to_dev(pool), to_dev(pool.copy())
    table = ops.rope_cos_sin_cache(P, rot, BASE)
    ops.paged_kv_write_rope(dq, dk, dv, kc, vc, to_dev(case.slot_mapping), to_dev(pos), table)
    torch.cuda.synchronize()
    ref = rope.rope_kv_write(case.q, case.k, case.v, pool, pool.copy(), case.slot_mapping, pos, bs, rot, BASE, dtype)
    return (dq, dk, kc, vc), ref, pos


def fp32_term(x, pos, rot, dtype, base=BASE):
    """4 fp32 ulps of |x1 c| + |x2 s| per rotated element (0 past rot_dim)."""
    xa = np.abs(oracle.upcast(x, dtype))
    tab = np.abs(rope.cos_sin_table(int(np.max(pos)) + 1, rot, base))[np.asarray(pos)][:, None, :]
    h = rot // 2
    m1 = xa[..., :h] * tab[..., :h] + xa[..., h:rot] * tab[..., h:]
    m2 = xa[..., h:rot] * tab[..., :h] + xa[..., :h] * tab[..., h:]
    out = np.zeros_like(xa)
    out[..., :h], out[..., h:rot] = m1, m2
    return 4 * 2.0 ** -24 * out


def check_rotated(gpu_t, ref_bits, x, pos, rot, dtype, what, base=BASE):
    ref64 = rope.rotate(x, pos, rot, base, dtype)
    bound = fp32_term(x, pos, rot, dtype, base)
    if dtype == wl.BF16:
        g = to_host_bits(gpu_t)
        err = np.abs(wl.bf16_bits_to_f32(g).astype(np.float64) - ref64)
        bound = bound + bf16_ulp(ref64)
        rate = (g == ref_bits).mean()
        assert rate > 0.999, f"{what}: exact-match rate {rate:.5f}"
    else:
        err = np.abs(to_host_f64(gpu_t) - ref64)
        bound = bound + 2.0 ** -24 * np.abs(ref64)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{what}: {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"


@pytest.mark.parametrize("dtype,rot", [(wl.BF16, 128), (wl.F32, 128), (wl.BF16, 64), (wl.F32, 32)])
def test_fused_rope_write(dtype, rot):
    case = wl.make_case(3, num_seqs=4, lens_fixed=(1, 63, 130, 300), dtype=dtype)
    (dq, dk, kc, vc), (qr, kr, okc, ovc), pos = run_fused(case, dtype, rot)
    bs = case.spec.block_size
    check_rotated(dq, qr, case.q, pos, rot, dtype, "q")
    check_rotated(dk, kr, case.k, pos, rot, dtype, "k")
    # dims past rot_dim pass through bit for bit
    np.testing.assert_array_equal(to_host_bits(dq)[..., rot:], case.q[..., rot:])
    np.testing.assert_array_equal(to_host_bits(dk)[..., rot:], case.k[..., rot:])
    # the pool holds exactly the in-place k and the input v; other slots untouched
    gk, gv = to_host_bits(kc), to_host_bits(vc)
    k_inplace = to_host_bits(dk)
    written = set()
    for t, s in enumerate(case.slot_mapping):
        s = int(s)
        np.testing.assert_array_equal(gk[s // bs, :, s % bs], k_inplace[t])
        np.testing.assert_array_equal(gv[s // bs, :, s % bs], case.v[t])
        written.add(s)
    for s in range(gk.shape[0] * bs):
        if s not in written:
            row = gk[s // bs, :, s % bs]
            assert np.isnan(wl.bf16_bits_to_f32(row) if dtype == wl.BF16 else row).all()


def test_negative_slots_rotate_but_write_nothing():
    case = wl.make_case(3, num_seqs=2, lens_fixed=(5, 9))
    case.slot_mapping[::2] = -1
    (dq, dk, kc, vc), (qr, kr, okc, ovc), pos = run_fused(case, wl.BF16, 128)
    check_rotated(dk, kr, case.k, pos, 128, wl.BF16, "k")
    gk = to_host_bits(kc)
    bs = case.spec.block_size
    for t, s in enumerate(case.slot_mapping):
        if s >= 0:
            np.testing.assert_array_equal(gk[s // bs, :, s % bs], to_host_bits(dk)[t])
    assert np.isnan(wl.bf16_bits_to_f32(to_host_bits(vc))).sum() == \
        np.isnan(wl.bf16_bits_to_f32(ovc)).sum()


def test_decode_over_rope_written_cache():
    # decode-step shape: every history row and the new row written through the
    # fused op at its own position, then a split decode of the rotated query
    spec_case = wl.make_case(2, batch=5, ctx_min=1, ctx_max=400, max_blocks_per_seq=25)
    bs, Hq, Hkv, d = 16, 32, 8, 128
    ctx = spec_case.context_lens
    tables = spec_case.block_tables
    slots, pos = [], []
    for b in range(len(ctx)):
        for p in range(int(ctx[b])):
            slots.append(int(tables[b, p // bs]) * bs + p % bs)
            pos.append(p)
    slots, pos = np.array(slots, np.int32), np.array(pos, np.int32)
    rng = np.random.default_rng(9)
    T = len(slots)
    k = wl.f32_to_bf16_bits(rng.normal(0, 1, (T, Hkv, d)).astype(np.float32))
    v = wl.f32_to_bf16_bits(rng.normal(0, 1, (T, Hkv, d)).astype(np.float32))
    # each sequence's query sits at its last position: rotate it with a one-row
    # q per written row (only the last row of each sequence is used)
    q_rows = wl.f32_to_bf16_bits(rng.normal(0, 1, (T, Hq, d)).astype(np.float32))
    pool = wl.empty_pool(spec_case.num_blocks, Hkv, bs, d, wl.BF16)
    dq, dk, dv = to_dev(q_rows), to_dev(k), to_dev(v)
    kc, vc = to_dev(pool), to_dev(pool.copy())
    table = ops.rope_cos_sin_cache(512, d, BASE)
    ops.paged_kv_write_rope(dq, dk, dv, kc, vc, to_dev(slots), to_dev(pos), table)
    last = np.cumsum(ctx.astype(np.int64)) - 1
    q_dev = dq[torch.from_numpy(last).cuda()].contiguous()
    ps = 64
    po, pl = ops.paged_attention_decode(q_dev, kc, vc, to_dev(tables), to_dev(ctx), spec_case.max_context_len,
                                        1 / np.sqrt(d), ps)
    out, lse = ops.paged_attention_reduce(po, pl, to_dev(ctx), ps, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    qr, kr, okc, ovc = rope.rope_kv_write(q_rows, k, v, pool, pool.copy(), slots, pos, bs, d, BASE, wl.BF16)
    ref_out, ref_lse = oracle.decode(qr[last], okc, ovc, tables, ctx, bs, 1 / np.sqrt(d), wl.BF16)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, wl.BF16, "decode after fused RoPE write")


def test_fused_rope_write_workload_full_size():
    """All of workload 3's prompt rows (16 sequences, 17,202 rows at its seed)
    in the benchmark's launch configuration: bf16, rot_dim = head_dim, a table
    of max_seqlen positions.  Every rotated element within the bar; the pool
    holds exactly the in-place k and the input v at each slot, NaN elsewhere."""
    case = wl.make_case(3)
    d, bs = case.spec.head_dim, case.spec.block_size
    (dq, dk, kc, vc), (qr, kr, _, _), pos = run_fused(case, wl.BF16, d, P=case.max_seqlen)
    check_rotated(dq, qr, case.q, pos, d, wl.BF16, "q")
    check_rotated(dk, kr, case.k, pos, d, wl.BF16, "k")
    slots = case.slot_mapping.astype(np.int64)
    assert (slots >= 0).all()
    want_k = wl.empty_pool(case.num_blocks, case.spec.num_kv_heads, bs, d, wl.BF16)
    want_v = want_k.copy()
    want_k[slots // bs, :, slots % bs] = to_host_bits(dk)
    want_v[slots // bs, :, slots % bs] = case.v
    np.testing.assert_array_equal(to_host_bits(kc), want_k)
    np.testing.assert_array_equal(to_host_bits(vc), want_v)
