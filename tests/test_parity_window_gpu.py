"""GPU parity of the sliding-window calls against the fp64 CPU oracle (C ABI).

A query at position p keeps positions max(0, p - W + 1) .. p.  Decode is
checked single-pass and split (the reduce merges the empty partials of the
partitions wholly before the window), prefill and paged prefill on ragged
sequences, each on the MFMA and the vector kernels.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def decode_window(case, ps, window):
    q, kc, vc = to_dev(case.q), to_dev(case.k_cache), to_dev(case.v_cache)
    bt, cl = to_dev(case.block_tables), to_dev(case.context_lens)
    if case.slot_mapping.size:
        ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    if ps:
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, window=window)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, window=window)
    torch.cuda.synchronize()
    return to_host_f64(out), to_host_f64(lse)


def decode_oracle(case, window):
    bs = case.spec.block_size
    kc, vc = case.k_cache, case.v_cache
    if case.slot_mapping.size:
        kc, vc = oracle.kv_write(kc, vc, case.k_new, case.v_new, case.slot_mapping, bs)
    return oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, bs, case.scale, case.spec.dtype,
                         window=window)


DECODE = {
    "bf16_g4_bs16": (2, dict(batch=6, ctx_min=1, ctx_max=600, max_blocks_per_seq=38)),
    "bf16_g8_bs32": (2, dict(batch=5, num_q_heads=16, num_kv_heads=2, block_size=32, ctx_min=1, ctx_max=500,
                             max_blocks_per_seq=16)),
    "f32_d64": (1, {}),
}


@pytest.mark.parametrize("name", sorted(DECODE))
@pytest.mark.parametrize("window", [1, 17, 100, 4096])
def test_window_decode(name, window):
    cfg, over = DECODE[name]
    case = wl.make_case(cfg, **over)
    ref_out, ref_lse = decode_oracle(case, window)
    for ps in (0, 64):
        out, lse = decode_window(case, ps, window)
        assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"{name} window={window} ps={ps}")


def test_window_decode_vector_kernel():
    cfg, over = DECODE["bf16_g4_bs16"]
    case = wl.make_case(cfg, **over)
    ref_out, ref_lse = decode_oracle(case, 33)
    try:
        ops.set_force_vector_path(True)
        for ps in (0, 64):
            out, lse = decode_window(case, ps, 33)
            assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"vector ps={ps}")
    finally:
        ops.set_force_vector_path(False)


PREFILL = {
    "bf16_g4": dict(num_seqs=4, lens_fixed=(1, 63, 130, 300)),
    "bf16_g1": dict(num_seqs=3, lens_fixed=(17, 64, 200), num_q_heads=2, num_kv_heads=2),
    "f32_d64": dict(dtype=wl.F32, num_seqs=3, lens_fixed=(5, 40, 90), num_q_heads=4, num_kv_heads=2,
                    head_dim=64),
}


@pytest.mark.parametrize("name", sorted(PREFILL))
@pytest.mark.parametrize("window", [1, 33, 64, 100])
def test_window_prefill(name, window):
    case = wl.make_case(3, **PREFILL[name])
    for vector in (False, True):
        try:
            ops.set_force_vector_path(vector)
            out, lse = ops.varlen_causal_prefill(to_dev(case.q), to_dev(case.k), to_dev(case.v),
                                                 to_dev(case.cu_seqlens), case.max_seqlen, case.scale, window=window)
            torch.cuda.synchronize()
        finally:
            ops.set_force_vector_path(False)
        ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype,
                                          window=window)
        assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype,
                      f"{name} window={window} vector={vector}")


PAGED = {
    "g4_bs16": dict(num_seqs=4, prefix_fixed=(0, 7, 100, 300), chunk_fixed=(5, 64, 33, 200)),
    "g1_bs8": dict(num_seqs=3, prefix_fixed=(3, 40, 129), chunk_fixed=(17, 64, 150), num_q_heads=2,
                   num_kv_heads=2, block_size=8),
}


@pytest.mark.parametrize("name", sorted(PAGED))
@pytest.mark.parametrize("window", [1, 45, 128, 300])
def test_window_paged_prefill(name, window):
    case = wl.make_case(6, **PAGED[name])
    bs = case.spec.block_size
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    out, lse = ops.paged_prefill(to_dev(case.q), kc, vc, to_dev(case.block_tables), to_dev(case.cu_seqlens_q),
                                 to_dev(case.context_lens), case.max_seqlen_q, case.max_context_len, case.scale,
                                 window=window)
    torch.cuda.synchronize()
    okc, ovc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    ref_out, ref_lse = oracle.paged_prefill(case.q, okc, ovc, case.block_tables, case.cu_seqlens_q,
                                            case.context_lens, bs, case.scale, case.spec.dtype, window=window)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"{name} window={window}")
