"""GPU parity of decode with the step's cache write folded in (C ABI).

paged_attention_decode_append must leave exactly the pools that
paged_kv_write + paged_attention_decode leave, and return exactly their
outputs (bit for bit: the same kernels read the same bytes), on the MFMA and
vector kernels, single pass and split, with and without a sliding window, for
bf16, f32 and E4M3 pools; and agree with the oracle's write + decode.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


def two_launch(case, ps, window, **fp8):
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping), **fp8)
    res = decode(case, kc, vc, ps, window, **fp8)
    return res, kc, vc


def one_launch(case, ps, window, **fp8):
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    res = decode(case, kc, vc, ps, window, k_new=to_dev(case.k_new), v_new=to_dev(case.v_new), **fp8)
    return res, kc, vc


def decode(case, kc, vc, ps, window, **kw):
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    if ps:
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, window=window,
                                            **kw)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, window=window)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, window=window,
                                              **kw)
    torch.cuda.synchronize()
    return out, lse


CASES = {
    "bf16_g4_bs16": (2, dict(batch=6, ctx_min=1, ctx_max=600, max_blocks_per_seq=38)),
    "bf16_g8_bs32": (2, dict(batch=5, num_q_heads=16, num_kv_heads=2, block_size=32, ctx_min=1, ctx_max=500,
                             max_blocks_per_seq=16)),
    "f32_d64": (1, {}),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("vector", [False, True])
def test_append_equals_write_then_decode(name, vector):
    cfg, over = CASES[name]
    case = wl.make_case(cfg, **over)
    try:
        ops.set_force_vector_path(vector)
        for ps in (0, 64):
            for window in (0, 100):
                (o2, l2), kc2, vc2 = two_launch(case, ps, window)
                (o1, l1), kc1, vc1 = one_launch(case, ps, window)
                what = f"{name} vector={vector} ps={ps} window={window}"
                np.testing.assert_array_equal(to_host_bits(kc1), to_host_bits(kc2), err_msg=what)
                np.testing.assert_array_equal(to_host_bits(vc1), to_host_bits(vc2), err_msg=what)
                np.testing.assert_array_equal(to_host_bits(o1), to_host_bits(o2), err_msg=what)
                np.testing.assert_array_equal(to_host_bits(l1), to_host_bits(l2), err_msg=what)
    finally:
        ops.set_force_vector_path(False)
    bs = case.spec.block_size
    ek, ev = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    ref_out, ref_lse = oracle.decode(case.q, ek, ev, case.block_tables, case.context_lens, bs, case.scale,
                                     case.spec.dtype)
    (o1, l1), _, _ = one_launch(case, 64, 0)
    assert_parity(to_host_f64(o1), to_host_f64(l1), ref_out, ref_lse, case.spec.dtype, f"{name} vs oracle")


def test_append_empty_sequence_writes_nothing():
    case = wl.make_case(2, batch=4, ctx_min=1, ctx_max=80, max_blocks_per_seq=6)
    case.context_lens[1] = 0
    case.slot_mapping[1] = -1
    (o2, l2), kc2, vc2 = two_launch(case, 16, 0)
    (o1, l1), kc1, vc1 = one_launch(case, 16, 0)
    np.testing.assert_array_equal(to_host_bits(kc1), to_host_bits(kc2))
    np.testing.assert_array_equal(to_host_bits(o1), to_host_bits(o2))
    assert np.isneginf(to_host_f64(l1)[1]).all()


def fp8_split(case):
    """History rows (all but each sequence's last) as the case's pre-written
    pools; the last rows as the step's new tokens."""
    last = np.cumsum(case.context_lens.astype(np.int64)) - 1
    hist = np.ones(len(case.slot_mapping), bool)
    hist[last] = False
    return last, hist


def test_append_fp8_equals_write_then_decode():
    case = wl.make_case(8, batch=6, ctx_min=1, ctx_max=600, max_blocks_per_seq=38)
    last, hist = fp8_split(case)
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    sc = dict(k_scale=ks, v_scale=vs)
    kc0, vc0 = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new[hist]), to_dev(case.v_new[hist]), kc0, vc0,
                       to_dev(case.slot_mapping[hist]), **sc)
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    kn, vn = to_dev(case.k_new[last]), to_dev(case.v_new[last])
    for ps in (0, 64):
        kc2, vc2 = kc0.clone(), vc0.clone()
        ops.paged_kv_write(kn, vn, kc2, vc2, to_dev(case.slot_mapping[last]), **sc)
        kc1, vc1 = kc0.clone(), vc0.clone()
        res = []
        for kc, vc, extra in ((kc2, vc2, {}), (kc1, vc1, dict(k_new=kn, v_new=vn))):
            if ps:
                po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, **sc,
                                                    **extra)
                res.append(ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype))
            else:
                res.append(ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, **sc,
                                                      **extra))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(kc1.cpu().numpy(), kc2.cpu().numpy())
        np.testing.assert_array_equal(vc1.cpu().numpy(), vc2.cpu().numpy())
        np.testing.assert_array_equal(to_host_bits(res[1][0]), to_host_bits(res[0][0]))
        np.testing.assert_array_equal(to_host_bits(res[1][1]), to_host_bits(res[0][1]))
    okc, ovc = oracle.kv_write_fp8(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                                   case.spec.block_size, case.spec.dtype, case.k_scale, case.v_scale)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, case.spec.block_size,
                                     case.scale, case.spec.dtype, kv_dtype=oracle.E4M3, k_scale=case.k_scale,
                                     v_scale=case.v_scale)
    assert_parity(to_host_f64(res[1][0]), to_host_f64(res[1][1]), ref_out, ref_lse, case.spec.dtype, "fp8 vs oracle")
