"""Device-resident inputs that break the preconditions (C ABI): block ids
outside the pool, context lengths past max_context_len, cu_seqlens past
total_tokens, slots outside the pool.  The header promises the kernels skip or
clamp these without touching memory outside the buffers; the results of the
sequences concerned are unspecified, and every other sequence must come out
bit for bit as in a run without the bad entries (each sequence's work depends
only on its own inputs).
"""
import numpy as np
import pytest
import torch

from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import to_dev, to_host_bits

pytestmark = pytest.mark.gpu

BAD_IDS = (-3, 1 << 30)   # plus num_blocks + 7, set per pool


def _spoil_tables(tables, ctx, bs, num_blocks, seqs):
    bad = tables.copy()
    for k, b in enumerate(seqs):
        nblk = -(-int(ctx[b]) // bs)
        if nblk == 0:
            continue
        ids = (num_blocks + 7,) + BAD_IDS
        for j in range(0, nblk, 3):
            bad[b, j] = ids[(j // 3 + k) % 3]
    return bad


def _decode(case, tables, ctx, ps, **kw):
    q, kc, vc = to_dev(case.q), to_dev(case.k_cache), to_dev(case.v_cache)
    bt, cl = to_dev(tables), to_dev(ctx)
    if ps:
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, ps, **kw)
        out, lse = ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype)
    else:
        out, lse = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, **kw)
    torch.cuda.synchronize()
    return to_host_bits(out), to_host_bits(lse)


@pytest.mark.parametrize("ps", [0, 128])
def test_decode_skips_bad_block_ids_and_clamps_contexts(ps):
    case = wl.make_case(2, batch=10, ctx_min=30, ctx_max=900, max_blocks_per_seq=60, write_new_token=False)
    bs, NB = case.spec.block_size, case.num_blocks
    spoiled = (1, 4, 7)
    tables = _spoil_tables(case.block_tables, case.context_lens, bs, NB, spoiled)
    ctx = case.context_lens.copy()
    ctx[9] = case.max_context_len + 500          # past max_context_len: clamped
    clean = _decode(case, case.block_tables, case.context_lens, ps)
    dirty = _decode(case, tables, ctx, ps)
    keep = [b for b in range(10) if b not in spoiled and b != 9]
    for a, b in zip(dirty, clean):
        np.testing.assert_array_equal(a[keep], b[keep])


def test_decode_fp8_skips_bad_block_ids():
    case = wl.make_case(8, batch=8, ctx_fixed=(40, 300, 700, 1, 128, 900, 64, 500), max_blocks_per_seq=60)
    bs, NB = case.spec.block_size, case.num_blocks
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping), k_scale=ks,
                       v_scale=vs)
    spoiled = (2, 5)
    tables = _spoil_tables(case.block_tables, case.context_lens, bs, NB, spoiled)
    res = []
    for t in (case.block_tables, tables):
        q, bt, cl = to_dev(case.q), to_dev(t), to_dev(case.context_lens)
        po, pl = ops.paged_attention_decode(q, kc, vc, bt, cl, case.max_context_len, case.scale, 256,
                                            k_scale=ks, v_scale=vs)
        out, lse = ops.paged_attention_reduce(po, pl, cl, 256, out_dtype=q.dtype)
        torch.cuda.synchronize()
        res.append((to_host_bits(out), to_host_bits(lse)))
    keep = [b for b in range(8) if b not in spoiled]
    for a, b in zip(res[1], res[0]):
        np.testing.assert_array_equal(a[keep], b[keep])


def test_paged_prefill_skips_bad_block_ids():
    case = wl.make_case(6, num_seqs=5, prefix_fixed=(0, 100, 300, 64, 200), chunk_fixed=(40, 70, 120, 1, 90))
    bs, NB = case.spec.block_size, case.num_blocks
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    spoiled = (1, 3)
    tables = _spoil_tables(case.block_tables, case.context_lens, bs, NB, spoiled)
    res = []
    for t in (case.block_tables, tables):
        out, lse = ops.paged_prefill(to_dev(case.q), kc, vc, to_dev(t), to_dev(case.cu_seqlens_q),
                                     to_dev(case.context_lens), case.max_seqlen_q, case.max_context_len, case.scale)
        torch.cuda.synchronize()
        res.append((to_host_bits(out), to_host_bits(lse)))
    cu = case.cu_seqlens_q
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in range(5) if s not in spoiled])
    for a, b in zip(res[1], res[0]):
        np.testing.assert_array_equal(a[rows], b[rows])


def test_varlen_prefill_clamps_cu_seqlens():
    case = wl.make_case(3, num_seqs=4, lens_fixed=(50, 130, 7, 200))
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    clean_out, clean_lse = ops.varlen_causal_prefill(q, k, v, to_dev(case.cu_seqlens), case.max_seqlen, case.scale)
    cu = case.cu_seqlens.copy()
    cu[2] = case.total_tokens + 1000            # sequence 1 runs past the packed rows (clamped), 2 is empty
    out, lse = ops.varlen_causal_prefill(q, k, v, to_dev(cu), case.max_seqlen, case.scale)
    torch.cuda.synchronize()
    rows = np.arange(0, int(case.cu_seqlens[1]))   # sequence 0
    np.testing.assert_array_equal(to_host_bits(out)[rows], to_host_bits(clean_out)[rows])
    np.testing.assert_array_equal(to_host_bits(lse)[rows], to_host_bits(clean_lse)[rows])


def test_kv_write_skips_slots_outside_the_pool():
    case = wl.make_case(2, batch=6, ctx_min=10, ctx_max=200, max_blocks_per_seq=13)
    bs, NB = case.spec.block_size, case.num_blocks
    slots = case.slot_mapping.copy()
    slots[1] = NB * bs + 5
    slots[3] = -(1 << 30)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(slots))
    torch.cuda.synchronize()
    want_k, want_v = case.k_cache.copy(), case.v_cache.copy()
    for t, s in enumerate(slots):
        if 0 <= s < NB * bs:
            want_k[s // bs, :, s % bs] = case.k_new[t]
            want_v[s // bs, :, s % bs] = case.v_new[t]
    np.testing.assert_array_equal(to_host_bits(kc), want_k)
    np.testing.assert_array_equal(to_host_bits(vc), want_v)
