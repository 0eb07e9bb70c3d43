"""GPU parity at the limits the header states (C ABI): 65535 sequences in one
launch, and 65535 split-KV partitions of one sequence.

At 65535 sequences the decode takes its per-sequence grid (the balanced flat
order stops at 1024 sequences) with the sequence dimension full, single pass
and split with the merge; the varlen and paged prefill take 65535 short
sequences (empty ones among them).  At 65535 partitions (a context of
1,048,560 positions in 16-position partitions) the merge takes its general
kernel and the single pass one workgroup per (sequence, KV head) over a
million keys.  Every output is compared with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

MAX_SEQS = 65535
MAX_PARTS = 65535


def decode(case, ps, window=0):
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    if case.slot_mapping.size:
        ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    maxctx = case.max_context_len
    if ps:
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, case.scale, ps, window=window)
        assert po.shape[2] == ops.num_partitions(maxctx, ps)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, window=window)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, case.scale, window=window)
    torch.cuda.synchronize()
    return to_host_f64(out), to_host_f64(lse)


def oracle_decode(case, window=0):
    bs = case.spec.block_size
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    return oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, bs, case.scale, case.spec.dtype,
                         window=window)


def test_decode_at_65535_sequences():
    print("decode, 65535 sequences", flush=True)
    case = wl.make_case(2, batch=MAX_SEQS, num_q_heads=4, num_kv_heads=2, ctx_min=0, ctx_max=40,
                        max_blocks_per_seq=3)
    assert (case.context_lens == 0).any() and case.max_context_len == 40
    ref_out, ref_lse = oracle_decode(case)
    for ps in (0, 16):
        out, lse = decode(case, ps)
        assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"65535 sequences ps={ps}")


def test_decode_at_65535_partitions():
    print("decode, 65535 partitions", flush=True)
    ctx = (MAX_PARTS * 16, 300001)
    case = wl.make_case(2, batch=2, ctx_fixed=ctx, num_q_heads=4, num_kv_heads=1, num_blocks=None,
                        pool_factor=1.0, max_blocks_per_seq=MAX_PARTS)
    assert ops.num_partitions(case.max_context_len, 16) == MAX_PARTS
    for window in (0, 1000):
        ref_out, ref_lse = oracle_decode(case, window)
        for ps in (16, 0):
            out, lse = decode(case, ps, window)
            assert_parity(out, lse, ref_out, ref_lse, case.spec.dtype, f"65535 partitions ps={ps} window={window}")


def test_prefill_at_65535_sequences():
    print("varlen prefill, 65535 sequences", flush=True)
    case = wl.make_case(3, num_seqs=MAX_SEQS, num_q_heads=4, num_kv_heads=2, len_min=0, len_max=5)
    lens = np.diff(case.cu_seqlens)
    assert (lens == 0).any()
    out, lse = ops.varlen_causal_prefill(to_dev(case.q), to_dev(case.k), to_dev(case.v), to_dev(case.cu_seqlens),
                                         case.max_seqlen, case.scale)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, case.spec.dtype)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, "65535 sequences")


def test_paged_prefill_at_65535_sequences():
    print("paged prefill, 65535 sequences", flush=True)
    case = wl.make_case(6, num_seqs=MAX_SEQS, num_q_heads=4, num_kv_heads=2, prefix_min=0, prefix_max=20,
                        chunk_min=0, chunk_max=4)
    bs = case.spec.block_size
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    out, lse = ops.paged_prefill(to_dev(case.q), kc, vc, to_dev(case.block_tables), to_dev(case.cu_seqlens_q),
                                 to_dev(case.context_lens), case.max_seqlen_q, case.max_context_len, case.scale)
    torch.cuda.synchronize()
    okc, ovc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    ref_out, ref_lse = oracle.paged_prefill(case.q, okc, ovc, case.block_tables, case.cu_seqlens_q,
                                            case.context_lens, bs, case.scale, case.spec.dtype)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, "65535 sequences")
