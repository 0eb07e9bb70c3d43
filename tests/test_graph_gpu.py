"""The decode step (cache write folded in, split decode, merge) and a varlen
prefill captured in a HIP graph (C ABI through the binding): every replay
gives bit for bit what the eager calls give, with the outputs refilled with
NaN by eager work between replays and the queries changed in place before the
last one.  The calls record no memset and keep no state between launches.
"""
import numpy as np
import pytest
import torch

from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def test_decode_step_and_prefill_replay_in_a_graph():
    dec = wl.make_case(2, batch=8, ctx_min=1, ctx_max=1200, max_blocks_per_seq=80)
    pre = wl.make_case(3, num_seqs=4, len_min=1, len_max=300)
    ps = 256
    B, Hq, d = dec.q.shape
    P = ops.num_partitions(dec.max_context_len, ps)
    q, kc, vc = to_dev(dec.q), to_dev(dec.k_cache), to_dev(dec.v_cache)
    bt, cl, kn, vn = to_dev(dec.block_tables), to_dev(dec.context_lens), to_dev(dec.k_new), to_dev(dec.v_new)
    pq, pk, pv, pcu = to_dev(pre.q), to_dev(pre.k), to_dev(pre.v), to_dev(pre.cu_seqlens)
    po = torch.empty((B, Hq, P, d), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, Hq, P), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    p_out = torch.empty_like(pq)
    p_lse = torch.empty((pre.total_tokens, pre.spec.num_q_heads), dtype=torch.float32, device="cuda")
    results = (out, lse, p_out, p_lse)

    def step():
        ops.paged_attention_decode(q, kc, vc, bt, cl, dec.max_context_len, dec.scale, ps, part_out=po, part_lse=pl,
                                   k_new=kn, v_new=vn)
        ops.paged_attention_reduce(po, pl, cl, ps, out=out, lse=lse)
        ops.varlen_causal_prefill(pq, pk, pv, pcu, pre.max_seqlen, pre.scale, out=p_out, lse=p_lse)

    def snapshot():
        torch.cuda.synchronize()
        return [t.contiguous().view(torch.uint8).cpu().numpy() for t in results]

    def refill():
        for t in results:
            t.fill_(float("nan"))

    # eager results for the original queries and for a second set
    step()
    want1 = snapshot()
    q_orig, pq_orig = q.clone(), pq.clone()
    rng = np.random.default_rng(5)
    q2 = torch.from_numpy(wl.f32_to_bf16_bits(rng.standard_normal(dec.q.shape).astype(np.float32)).view(np.int16))
    pq2 = torch.from_numpy(wl.f32_to_bf16_bits(rng.standard_normal(pre.q.shape).astype(np.float32)).view(np.int16))
    q2, pq2 = q2.view(torch.bfloat16).cuda(), pq2.view(torch.bfloat16).cuda()
    q.copy_(q2)
    pq.copy_(pq2)
    step()
    want2 = snapshot()
    q.copy_(q_orig)
    pq.copy_(pq_orig)

    # capture (after a warm-up on a side stream, as torch's capture expects)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        refill()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, want1):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}")
    refill()
    q.copy_(q2)
    pq.copy_(pq2)
    graph.replay()
    for a, b in zip(snapshot(), want2):
        np.testing.assert_array_equal(a, b, err_msg="replay with changed queries")
