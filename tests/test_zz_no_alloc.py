"""paged_attention_decode_noalloc: the split decode and its merge with the
partials in the library's own per-GPU scratch (nothing allocated by the call).

Through the C ABI it must give exactly what paged_attention_decode (split) +
paged_attention_reduce give with caller-owned partials - the same kernels, so
bit for bit - on two calls in a row, the second smaller than the first, and
stay within the parity bar of the oracle.  Sizes past the scratch are refused
before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_f64


def _reference(case, ps, window):
    q, kc, vc = to_dev(case.q), to_dev(case.k_cache), to_dev(case.v_cache)
    bt, cl = to_dev(case.block_tables), to_dev(case.context_lens)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, window=window)
    out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, window=window)
    return (q, kc, vc, bt, cl), out, lse


@pytest.mark.gpu
@pytest.mark.parametrize("window", [0, 300])
def test_noalloc_matches_split_decode_twice(window):
    big = wl.make_case(2, batch=24, ctx_min=1, ctx_max=2048, max_blocks_per_seq=128)
    small = wl.make_case(2, seed=77, batch=5, ctx_min=1, ctx_max=700, max_blocks_per_seq=44)
    for case, ps in ((big, 256), (small, 128)):
        (q, kc, vc, bt, cl), ref_out, ref_lse = _reference(case, ps, window)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
        ops.paged_attention_decode_noalloc(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, out, lse,
                                           window=window)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), (ps, window)
        assert torch.equal(lse, ref_lse), (ps, window)
        ek, ev = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                                 case.spec.block_size)
        o_out, o_lse = oracle.decode(case.q, ek, ev, case.block_tables, case.context_lens, case.spec.block_size,
                                     case.scale, case.spec.dtype, window=window)
        assert_parity(to_host_f64(out), to_host_f64(lse), o_out, o_lse, case.spec.dtype, f"noalloc ps={ps}")


@pytest.mark.gpu
def test_noalloc_f32_vector_kernels_twice():
    # fp32 queries and pools at head_dim 64 (the vector decode kernel and the
    # fp32 merge), GQA group 4, 32-token blocks, under a window on the second call
    big = wl.make_case(1, batch=9, ctx_fixed=None, ctx_min=1, ctx_max=900, num_q_heads=8, num_kv_heads=2,
                       block_size=32, num_blocks=None, max_blocks_per_seq=29)
    small = wl.make_case(1, seed=78, batch=3, ctx_fixed=(1, 64, 300), num_q_heads=8, num_kv_heads=2,
                         block_size=32, num_blocks=None, max_blocks_per_seq=10)
    for case, ps, window in ((big, 128, 0), (small, 64, 100)):
        (q, kc, vc, bt, cl), ref_out, ref_lse = _reference(case, ps, window)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
        ops.paged_attention_decode_noalloc(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, out, lse,
                                           window=window)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), (ps, window)
        assert torch.equal(lse, ref_lse), (ps, window)
        ek, ev = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                                 case.spec.block_size)
        o_out, o_lse = oracle.decode(case.q, ek, ev, case.block_tables, case.context_lens, case.spec.block_size,
                                     case.scale, case.spec.dtype, window=window)
        assert_parity(to_host_f64(out), to_host_f64(lse), o_out, o_lse, case.spec.dtype, f"noalloc f32 ps={ps}")


@pytest.mark.gpu
def test_noalloc_in_a_hip_graph():
    # the call as its callers make it under graph capture: captured once, then
    # replayed three times with eager work (refilling the outputs with NaN)
    # between the replays; every replay equals the two-call path bit for bit
    case = wl.make_case(2, seed=91, batch=12, ctx_min=1, ctx_max=1500, max_blocks_per_seq=94)
    ps = 256
    (q, kc, vc, bt, cl), ref_out, ref_lse = _reference(case, ps, 0)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    # an eager call first, so the scratch address is looked up outside the capture
    ops.paged_attention_decode_noalloc(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.paged_attention_decode_noalloc(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, out, lse)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), r
        assert torch.equal(lse, ref_lse), r
    del g


def test_noalloc_refuses_partials_past_the_scratch():
    # 4 sequences x 32 heads x 2048 partitions x 129 floats = 135 MB > 32 MiB:
    # refused by the host checks, nothing launched (no GPU needed)
    lib = ops.load_library()
    p = ctypes.c_void_p(16)
    rc = lib.paged_attention_decode_noalloc(p, p, p, p, p, p, p, 4, 32, 8, 128, 16, 8192, 40960, 64, 131072,
                                            0.088, 0, 1, None)
    assert rc == 1 and "scratch" in lib.pa_last_error().decode()
    # partition_size 0 is not a split call
    rc = lib.paged_attention_decode_noalloc(p, p, p, p, p, p, p, 4, 32, 8, 128, 16, 8, 100, 0, 128, 0.088, 0, 1,
                                            None)
    assert rc == 1
