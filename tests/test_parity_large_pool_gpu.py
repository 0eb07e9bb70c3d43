"""Pools past 32 GiB: every call that addresses a paged pool, with the live
blocks placed beyond 2^35 bytes into the pools (C ABI).

A serving pool fills most of the 288 GB of HBM, so a block's byte offset runs
far past 2^32 (a 32-bit byte offset) and its 16-byte chunk index past 2^31 (a
32-bit chunk index).  Each case is built small, its blocks copied to block ids
base .. base + NB - 1 of two 34 GiB pools (K and V) whose other bytes are 0xFF
(NaN in bf16, f32 and E4M3), and its tables and slots shifted by base.  The
outputs must be bit-identical to the same call on the compact pool (the work
split depends only on logical positions, not on block ids), and within the
oracle's tolerance; written blocks must equal the oracle's write bit for bit
and the bytes around them stay 0xFF.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

POOL_BYTES = (1 << 35) + (64 << 20)   # 32 GiB + 64 MiB per pool
OFFSET = (1 << 35) + (16 << 20)       # live blocks start past 32 GiB


@pytest.fixture(scope="module")
def big_pools():
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * POOL_BYTES + (4 << 30):
        pytest.skip(f"needs {2 * POOL_BYTES / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    print(f"allocating two pools of {POOL_BYTES / 2**30:.2f} GiB", flush=True)
    k = torch.empty(POOL_BYTES, dtype=torch.uint8, device="cuda")
    v = torch.empty(POOL_BYTES, dtype=torch.uint8, device="cuda")
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def _torch_dtype(a):
    return {np.uint16: torch.bfloat16, np.float32: torch.float32, np.uint8: torch.uint8}[a.dtype.type]


def relocate(big, small):
    """View `big` as a pool of small's block shape and dtype, refill it with
    0xFF, and copy small's blocks to ids base .. base + NB - 1; returns the
    view and base."""
    big.fill_(0xFF)
    NB = small.shape[0]
    block_bytes = small[0].nbytes
    base = -(-OFFSET // block_bytes)
    total = (POOL_BYTES // block_bytes)
    assert base + NB <= total
    view = big[:total * block_bytes].view(_torch_dtype(small)).view((total,) + small.shape[1:])
    view[base:base + NB] = to_dev(small)
    return view, base


def shift_tables(tables, base):
    t = tables.astype(np.int64)
    return np.where(t >= 0, t + base, t).astype(np.int32)


def shift_slots(slots, base, bs):
    s = slots.astype(np.int64)
    return np.where(s >= 0, s + base * bs, s).astype(np.int32)


def fp8_scales(case):
    return (torch.tensor([case.k_scale], dtype=torch.float32, device="cuda"),
            torch.tensor([case.v_scale], dtype=torch.float32, device="cuda"))


def decode_call(case, kc, vc, tables, ps, window, maxctx, append=False, scales=None):
    q, bt, cl = to_dev(case.q), to_dev(tables), to_dev(case.context_lens)
    kw = {}
    if scales is not None:
        kw = dict(k_scale=scales[0], v_scale=scales[1])
    if append:
        kw.update(k_new=to_dev(case.k_new), v_new=to_dev(case.v_new))
    if ps:
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, case.scale, ps, window=window, **kw)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, window=window)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, case.scale, window=window, **kw)
    torch.cuda.synchronize()
    return to_host_bits(out), to_host_bits(lse)


def check_written(view, base, oracle_pool, what):
    """The relocated blocks equal the oracle's pool, and the blocks just
    before and after them still hold 0xFF bytes."""
    NB = oracle_pool.shape[0]
    np.testing.assert_array_equal(to_host_bits(view[base:base + NB]), oracle_pool, err_msg=what)
    for blk in (base - 1, base + NB):
        if 0 <= blk < view.shape[0]:
            raw = view[blk].contiguous().view(torch.uint8).cpu().numpy()
            assert (raw == 0xFF).all(), f"{what}: block {blk} beside the live ones was written"


DECODE_CASES = {
    "bf16_mfma_g4_bs16": dict(batch=5, ctx_fixed=(1, 17, 300, 1000, 2048), num_q_heads=8, num_kv_heads=2,
                             max_blocks_per_seq=128),
    "bf16_mfma_g8_bs32": dict(batch=3, ctx_fixed=(40, 700, 1500), num_q_heads=16, num_kv_heads=2, block_size=32,
                             max_blocks_per_seq=48),
    "f32_d64_vector": dict(dtype=wl.F32, head_dim=64, batch=4, ctx_fixed=(1, 33, 250, 900), num_q_heads=4,
                           num_kv_heads=2, max_blocks_per_seq=64),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_past_32gib(big_pools, name):
    print("decode", name, flush=True)
    case = wl.make_case(2, **DECODE_CASES[name])
    bs = case.spec.block_size
    okc, ovc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    for append in (False, True):
        # the compact pool, written the same way
        kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
        if not append:
            ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
        # the relocated pool
        bk, base = relocate(big_pools[0], case.k_cache)
        bv, _ = relocate(big_pools[1], case.v_cache)
        big_tables = shift_tables(case.block_tables, base)
        if not append:
            ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), bk, bv,
                               to_dev(shift_slots(case.slot_mapping, base, bs)))
        for window in (0, 100):
            ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs,
                                             case.scale, case.spec.dtype, window=window)
            for ps in (0, 256):
                what = f"{name} append={append} window={window} ps={ps}"
                # the appended row goes in once per pool; later calls rewrite the same bytes
                small = decode_call(case, kc, vc, case.block_tables, ps, window, case.max_context_len, append)
                large = decode_call(case, bk, bv, big_tables, ps, window, case.max_context_len, append)
                np.testing.assert_array_equal(large[0], small[0], err_msg=what)
                np.testing.assert_array_equal(large[1], small[1], err_msg=what)
                out = wl.bf16_bits_to_f32(large[0]).astype(np.float64) if large[0].dtype == np.uint16 \
                    else large[0].astype(np.float64)
                assert_parity(out, large[1].astype(np.float64), ref_out, ref_lse, case.spec.dtype, what)
        check_written(bk, base, okc, f"{name} append={append} k")
        check_written(bv, base, ovc, f"{name} append={append} v")


def test_fp8_write_and_decode_past_32gib(big_pools):
    print("fp8 write and decode", flush=True)
    case = wl.make_case(8, batch=4, ctx_fixed=(1, 100, 700, 2000), num_q_heads=8, num_kv_heads=2,
                        max_blocks_per_seq=128)
    bs = case.spec.block_size
    okc, ovc = oracle.kv_write_fp8(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs,
                                   case.spec.dtype, case.k_scale, case.v_scale)
    scales = fp8_scales(case)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping),
                       k_scale=scales[0], v_scale=scales[1])
    bk, base = relocate(big_pools[0], case.k_cache)
    bv, _ = relocate(big_pools[1], case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), bk, bv,
                       to_dev(shift_slots(case.slot_mapping, base, bs)), k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    check_written(bk, base, okc, "fp8 k")
    check_written(bv, base, ovc, "fp8 v")
    big_tables = shift_tables(case.block_tables, base)
    for window in (0, 100):
        ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, case.scale,
                                         case.spec.dtype, window=window, kv_dtype=oracle.E4M3,
                                         k_scale=case.k_scale, v_scale=case.v_scale)
        for ps in (0, 512):
            what = f"fp8 window={window} ps={ps}"
            small = decode_call(case, kc, vc, case.block_tables, ps, window, case.max_context_len, scales=scales)
            large = decode_call(case, bk, bv, big_tables, ps, window, case.max_context_len, scales=scales)
            np.testing.assert_array_equal(large[0], small[0], err_msg=what)
            np.testing.assert_array_equal(large[1], small[1], err_msg=what)
            assert_parity(wl.bf16_bits_to_f32(large[0]).astype(np.float64), large[1].astype(np.float64), ref_out,
                          ref_lse, case.spec.dtype, what)


PAGED_PREFILL_CASES = {
    "bf16_mfma": dict(num_seqs=3, prefix_fixed=(0, 70, 400), chunk_fixed=(33, 128, 90), num_q_heads=8,
                      num_kv_heads=2),
    "bf16_mfma_bs8": dict(num_seqs=2, prefix_fixed=(5, 200), chunk_fixed=(64, 17), num_q_heads=4, num_kv_heads=2,
                          block_size=8),
    "f32_d64_vector": dict(dtype=wl.F32, head_dim=64, num_seqs=2, prefix_fixed=(9, 150), chunk_fixed=(20, 40),
                           num_q_heads=4, num_kv_heads=2),
}


@pytest.mark.parametrize("name", sorted(PAGED_PREFILL_CASES))
def test_paged_prefill_past_32gib(big_pools, name):
    print("paged prefill", name, flush=True)
    case = wl.make_case(6, **PAGED_PREFILL_CASES[name])
    bs = case.spec.block_size
    okc, ovc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    bk, base = relocate(big_pools[0], case.k_cache)
    bv, _ = relocate(big_pools[1], case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), bk, bv, to_dev(shift_slots(case.slot_mapping, base, bs)))
    torch.cuda.synchronize()
    check_written(bk, base, okc, f"{name} k")
    check_written(bv, base, ovc, f"{name} v")
    big_tables = shift_tables(case.block_tables, base)
    for window in (0, 50):
        ref_out, ref_lse = oracle.paged_prefill(case.q, okc, ovc, case.block_tables, case.cu_seqlens_q,
                                                case.context_lens, bs, case.scale, case.spec.dtype, window=window)
        res = []
        for (k, v, t) in ((kc, vc, case.block_tables), (bk, bv, big_tables)):
            out, lse = ops.paged_prefill(to_dev(case.q), k, v, to_dev(t), to_dev(case.cu_seqlens_q),
                                         to_dev(case.context_lens), case.max_seqlen_q, case.max_context_len,
                                         case.scale, window=window)
            torch.cuda.synchronize()
            res.append((out, lse))
        what = f"{name} window={window}"
        np.testing.assert_array_equal(to_host_bits(res[1][0]), to_host_bits(res[0][0]), err_msg=what)
        np.testing.assert_array_equal(to_host_bits(res[1][1]), to_host_bits(res[0][1]), err_msg=what)
        assert_parity(to_host_f64(res[1][0]), to_host_f64(res[1][1]), ref_out, ref_lse, case.spec.dtype, what)


def test_rope_write_past_32gib(big_pools):
    print("rope write", flush=True)
    case = wl.make_case(3, num_seqs=3, lens_fixed=(1, 70, 300), num_q_heads=8, num_kv_heads=2)
    bs, (T, Hq, d), Hkv = case.spec.block_size, case.q.shape, case.k.shape[1]
    pos = np.concatenate([np.arange(n) for n in np.diff(case.cu_seqlens)]).astype(np.int32)
    table = ops.rope_cos_sin_cache(4096, 128)
    pool = wl.empty_pool(case.num_blocks, Hkv, bs, d, wl.BF16)
    outs = []
    for big in (False, True):
        q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
        if big:
            kc, base = relocate(big_pools[0], pool)
            vc, _ = relocate(big_pools[1], pool)
            slots = shift_slots(case.slot_mapping, base, bs)
        else:
            kc, vc, base, slots = to_dev(pool), to_dev(pool.copy()), 0, case.slot_mapping
        ops.paged_kv_write_rope(q, k, v, kc, vc, to_dev(slots), to_dev(pos), table)
        torch.cuda.synchronize()
        outs.append((to_host_bits(q), to_host_bits(k), to_host_bits(kc[base:base + case.num_blocks]),
                     to_host_bits(vc[base:base + case.num_blocks])))
    for a, b, what in zip(outs[1], outs[0], ("q", "k", "k pool", "v pool")):
        np.testing.assert_array_equal(a, b, err_msg=what)
    # the pool holds the rotated k and the input v at each slot
    k_rot = outs[1][1]
    for t, s in enumerate(case.slot_mapping):
        np.testing.assert_array_equal(outs[1][2][s // bs, :, s % bs], k_rot[t])
        np.testing.assert_array_equal(outs[1][3][s // bs, :, s % bs], case.v[t])
