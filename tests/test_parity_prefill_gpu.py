"""GPU parity of varlen_causal_prefill against the fp64 CPU oracle, through the C ABI.

Shrunk workloads are compared on every output; the full Llama-3-8B varlen
workload (16 sequences, about 16.9k tokens) on a sample of heads.  Row 0 of
each sequence must return v_0 bit-exactly (this pins the cu_seqlens
boundaries), and the last row of each sequence must match a decode over a
paged pool written from the same K/V (cross-path).
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


def run_prefill(case):
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    cu = to_dev(case.cu_seqlens)
    out, lse = ops.varlen_causal_prefill(q, k, v, cu, case.max_seqlen, case.scale)
    torch.cuda.synchronize()
    return out, lse


PREFILL_CASES = {
    "ragged_small": dict(num_seqs=6, lens_fixed=(1, 63, 64, 65, 130, 300)),
    "single_seq": dict(num_seqs=1, lens_fixed=(257,)),
    "g8": dict(num_seqs=3, lens_fixed=(5, 100, 200), num_q_heads=16, num_kv_heads=2),
    "g1": dict(num_seqs=3, lens_fixed=(17, 64, 129), num_q_heads=4, num_kv_heads=4),
    # one head per workgroup, four 32-row waves: rows past the wave's diagonal
    # tile and waves wholly past the sequence end
    "g1_long": dict(num_seqs=4, lens_fixed=(1, 40, 200, 333), num_q_heads=2, num_kv_heads=2),
    "g2": dict(num_seqs=3, lens_fixed=(33, 96, 161), num_q_heads=8, num_kv_heads=4),
    "f32_d64": dict(dtype=wl.F32, num_seqs=4, lens_fixed=(1, 10, 33, 70), num_q_heads=4,
                    num_kv_heads=2, head_dim=64),
    "bf16_d64": dict(num_seqs=3, lens_fixed=(3, 40, 90), num_q_heads=4, num_kv_heads=2, head_dim=64),
    "f32_d128": dict(dtype=wl.F32, num_seqs=2, lens_fixed=(31, 77), num_q_heads=8, num_kv_heads=2),
    # fewer head columns than XCDs: 2 columns shared by 4 XCDs each, whole
    # sequences dealt to them (18 of near-equal length: the launcher deals when
    # the mean length is at least 0.8 of the longest) or q tiles interleaved
    # (3 uneven ones)
    "two_columns_dealt": dict(num_seqs=18, lens_fixed=(300, 290, 281, 299, 250, 300, 257, 264, 300, 295, 288,
                                                       270, 241, 300, 299, 262, 277, 300),
                              num_q_heads=8, num_kv_heads=1),
    "two_columns_interleaved": dict(num_seqs=3, lens_fixed=(700, 1, 333), num_q_heads=8, num_kv_heads=2),
    # one column over all 8 XCDs, 33 sequences dealt (one of them empty)
    "one_column_dealt": dict(num_seqs=33, lens_fixed=(0,) + tuple(190 + (7 * i) % 11 for i in range(32)),
                             num_q_heads=4, num_kv_heads=1),
}


@pytest.mark.parametrize("name", sorted(PREFILL_CASES))
def test_prefill_matches_oracle(name):
    case = wl.make_case(3, **PREFILL_CASES[name])
    out, lse = run_prefill(case)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, name)


def _growing_scores(case, rng, slope=0.3, q_len=4.0):
    """Rewrite q and k so that every query's scores grow along the keys: keys
    are slope * position along one unit direction u (plus a little noise),
    queries q_len * u.  Each 64-key tile then raises a row's max by about
    0.1 nats per key, past the lazy-rescale slack, so the running max and O are
    rescaled at nearly every tile."""
    d = case.spec.head_dim
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    cu = case.cu_seqlens.astype(np.int64)
    pos = np.concatenate([np.arange(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]).astype(np.float64)
    k = slope * pos[:, None, None] * u[None, None, :] + 0.01 * rng.standard_normal(case.k.shape)
    q = q_len * u[None, None, :] + 0.01 * rng.standard_normal(case.q.shape)
    case.k = wl.f32_to_bf16_bits(k.astype(np.float32))
    case.q = wl.f32_to_bf16_bits(q.astype(np.float32))
    return case


@pytest.mark.parametrize("lens", [(300, 700, 1030), (64, 65, 129)])
def test_prefill_growing_scores_rescale_every_tile(lens):
    case = _growing_scores(wl.make_case(3, num_seqs=len(lens), lens_fixed=lens), np.random.default_rng(5))
    out, lse = run_prefill(case)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype)
    assert ref_lse.max() > 0.09 * (max(lens) - 1)   # the scores really grow along the keys
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"growing {lens}")


@pytest.mark.parametrize("window", [1, 40, 100, 257])
def test_prefill_growing_scores_under_window(window):
    # the same growing scores under a sliding window: a row's first visible key
    # can lie in a later tile than the workgroup's first, so its running max
    # goes from -inf to finite mid-loop and then keeps growing
    lens = (300, 700, 1030)
    case = _growing_scores(wl.make_case(3, num_seqs=len(lens), lens_fixed=lens), np.random.default_rng(7))
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    out, lse = ops.varlen_causal_prefill(q, k, v, to_dev(case.cu_seqlens), case.max_seqlen, case.scale, window=window)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype,
                                      window=window)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype,
                  f"growing, window {window}")


@pytest.mark.parametrize("name", ["ragged_small", "g8"])
def test_prefill_vector_kernel_matches_oracle(name):
    case = wl.make_case(3, **PREFILL_CASES[name])
    try:
        ops.set_force_vector_path(True)
        out, lse = run_prefill(case)
    finally:
        ops.set_force_vector_path(False)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, name + " vector")


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_prefill_scale_sign_and_zero(scale):
    # a negative scale reverses which key scores highest; zero gives the plain
    # mean of the visible values
    import dataclasses
    case = dataclasses.replace(wl.make_case(3, **PREFILL_CASES["ragged_small"]), scale=scale)
    out, lse = run_prefill(case)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"scale={scale}")


def test_prefill_is_deterministic():
    # repeated launches on the same inputs give the same bits (no read of a
    # matrix-core result before it is ready, no LDS race between waves)
    case = wl.make_case(3, num_seqs=3, lens_fixed=(1, 100, 257))
    q, k, v, cu = to_dev(case.q), to_dev(case.k), to_dev(case.v), to_dev(case.cu_seqlens)
    runs = []
    for _ in range(3):
        out, lse = ops.varlen_causal_prefill(q, k, v, cu, case.max_seqlen, case.scale)
        torch.cuda.synchronize()
        runs.append((to_host_bits(out), to_host_bits(lse)))
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])


def test_prefill_row0_is_v0_bit_exact():
    case = wl.make_case(3, **PREFILL_CASES["ragged_small"])
    out, lse = run_prefill(case)
    ob = to_host_bits(out)
    lh = to_host_f64(lse)
    G = case.spec.num_q_heads // case.spec.num_kv_heads
    for s in range(case.spec.num_seqs):
        a = int(case.cu_seqlens[s])
        for h in range(case.spec.num_q_heads):
            assert ob[a, h].tobytes() == case.v[a, h // G].tobytes(), (s, h)
            _, l1, _ = oracle.attend(oracle.upcast(case.q[a, h], wl.BF16),
                                     oracle.upcast(case.k[a:a + 1, h // G], wl.BF16),
                                     oracle.upcast(case.v[a:a + 1, h // G], wl.BF16), case.scale)
            assert abs(lh[a, h] - l1) <= 1e-3


def test_prefill_leaves_uncovered_tokens_untouched():
    # cu_seqlens covering only part of the buffer: tokens outside are not written
    case = wl.make_case(3, **PREFILL_CASES["ragged_small"])
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    T = q.shape[0]
    cu = to_dev(np.array([0, 64, 129], np.int32))  # first two sequences only
    out = torch.full_like(q, 7.0)
    lse = torch.full((T, q.shape[1]), 7.0, device=q.device)
    ops.varlen_causal_prefill(q, k, v, cu, 65, case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out[129:] == 7.0) and torch.all(lse[129:] == 7.0)
    ref_out, ref_lse = oracle.prefill(case.q[:129], case.k[:129], case.v[:129],
                                      np.array([0, 64, 129]), case.scale, wl.BF16)
    assert_parity(to_host_f64(out[:129]), to_host_f64(lse[:129]), ref_out, ref_lse, wl.BF16, "partial")


def test_prefill_write_then_decode_cross_path():
    case = wl.make_case(3, num_seqs=4, lens_fixed=(1, 50, 128, 333))
    spec = case.spec
    out, lse = run_prefill(case)
    pk = wl.empty_pool(case.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim, spec.dtype)
    kc, vc = to_dev(pk), to_dev(pk.copy())
    ops.paged_kv_write(to_dev(case.k), to_dev(case.v), kc, vc, to_dev(case.slot_mapping))
    last = case.cu_seqlens[1:] - 1
    lens = np.diff(case.cu_seqlens).astype(np.int32)
    dout, dlse = ops.paged_attention_decode(to_dev(case.q[last]), kc, vc, to_dev(case.block_tables),
                                            to_dev(lens), int(lens.max()), case.scale)
    torch.cuda.synchronize()
    # the decode and the prefill agree with the oracle's decode of the same rows
    ek, ev = oracle.kv_write(pk, pk.copy(), case.k, case.v, case.slot_mapping, spec.block_size)
    ref_out, ref_lse = oracle.decode(case.q[last], ek, ev, case.block_tables, lens, spec.block_size,
                                     case.scale, spec.dtype)
    assert_parity(to_host_f64(dout), to_host_f64(dlse), ref_out, ref_lse, spec.dtype, "decode of prompt")
    assert_parity(to_host_f64(out)[last], to_host_f64(lse)[last], ref_out, ref_lse, spec.dtype,
                  "prefill last rows")


@pytest.mark.slow
def test_prefill_full_size_every_output():
    # workload 3 at full size (16 sequences, about 17k rows): every row of every head
    case = wl.make_case(3)
    out, lse = run_prefill(case)
    oh, lh = to_host_f64(out), to_host_f64(lse)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, wl.BF16)
    assert_parity(oh, lh, ref_out, ref_lse, wl.BF16, "workload 3, every (row, head)")
