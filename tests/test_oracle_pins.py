"""Pins for the fp64 CPU oracle (no GPU needed).

The oracle is checked against things other than itself: hand-worked closed
forms under tests/golden/ (each citing its passage), a library routine (torch's
CPU scaled_dot_product_attention in float64), invariants of the paging model
(paged equals unpaged, block permutation and block size do not matter), special
cases with exact answers (one key, a one-hot "needle", constant V), and a
pure-Python brute-force spelling on tiny inputs.  tests/test_oracle_mutants.py
plants mistakes in copies of the oracle and checks that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from attention_paged_kv_write_amd import workloads as wl




def load_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers that build inputs (no attention arithmetic here)
# ---------------------------------------------------------------------------
def page_contiguous(K, V, block_size, rng, extra_blocks=3, fill=np.nan):
    """Scatter contiguous [n, Hkv, d] K/V into a shuffled pool; returns pool + table row."""
    n, Hkv, d = K.shape
    nblk = -(-n // block_size)
    NB = nblk + extra_blocks
    ids = rng.permutation(NB)[:nblk].astype(np.int32)
    kp = np.full((NB, Hkv, block_size, d), fill, dtype=K.dtype)
    vp = np.full((NB, Hkv, block_size, d), fill, dtype=V.dtype)
    for p in range(n):
        kp[ids[p // block_size], :, p % block_size, :] = K[p]
        vp[ids[p // block_size], :, p % block_size, :] = V[p]
    return kp, vp, ids


def paged_batch(Ks, Vs, block_size, rng, extra_blocks=5, max_blocks=None):
    """Several sequences' contiguous K/V -> one shared shuffled pool + tables."""
    Hkv, d = Ks[0].shape[1], Ks[0].shape[2]
    nblks = [-(-K.shape[0] // block_size) for K in Ks]
    NB = sum(nblks) + extra_blocks
    perm = rng.permutation(NB).astype(np.int32)
    M = max_blocks or max(max(nblks), 1)
    tables = np.full((len(Ks), M), -1, dtype=np.int32)
    kp = np.full((NB, Hkv, block_size, d), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    c = 0
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        tables[b, :nblks[b]] = perm[c:c + nblks[b]]
        c += nblks[b]
        for p in range(K.shape[0]):
            kp[tables[b, p // block_size], :, p % block_size, :] = K[p]
            vp[tables[b, p // block_size], :, p % block_size, :] = V[p]
    ctx = np.array([K.shape[0] for K in Ks], dtype=np.int32)
    return kp, vp, tables, ctx


def sdpa_decode_reference(q, Ks, Vs, scale):
    """torch CPU float64 SDPA on contiguous K/V, K/V heads repeated per group."""
    B, Hq, d = q.shape
    outs, lses = [], []
    for b in range(B):
        K = torch.from_numpy(Ks[b].astype(np.float64)).permute(1, 0, 2)  # [Hkv, n, d]
        V = torch.from_numpy(Vs[b].astype(np.float64)).permute(1, 0, 2)
        G = Hq // K.shape[0]
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]       # [Hq, 1, d]
        o = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], scale=scale)[0, :, 0, :]
        s = (Q @ K.transpose(1, 2))[:, 0, :] * scale
        outs.append(o.numpy())
        lses.append(torch.logsumexp(s, dim=-1).numpy())
    return np.stack(outs), np.stack(lses)


def rand_f32(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


# ---------------------------------------------------------------------------
# golden closed forms
# ---------------------------------------------------------------------------
def test_golden_kv_write(golden_dir):
    g = load_golden(golden_dir, "kv_write_tiny.json")
    NB, H, bs, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    kp = np.zeros((NB, H, bs, d), dtype=np.float32)
    for blk in range(NB):
        for h in range(H):
            for off in range(bs):
                for e in range(d):
                    kp[blk, h, off, e] = 1000 * blk + 100 * h + 10 * off + e
    vp = kp + np.float32(0.5)
    kn = np.array(g["k_new"], dtype=np.float32)
    vn = np.array(g["v_new"], dtype=np.float32)
    slots = np.array(g["slot_mapping"], dtype=np.int32)
    kc, vc = oracle.kv_write(kp, vp, kn, vn, slots, bs)
    np.testing.assert_array_equal(kc, np.array(g["expected_k_pool"], dtype=np.float32))
    np.testing.assert_array_equal(vc, np.array(g["expected_v_pool"], dtype=np.float32))
    got = oracle.gather(kc, np.array(g["gather_table_row"]), g["gather_ctx"], bs)
    np.testing.assert_array_equal(got, np.array(g["expected_gather_k"], dtype=np.float32))


def test_golden_attention_closed_form(golden_dir):
    g = load_golden(golden_dir, "attention_closed_form.json")
    out, lse, probs = oracle.attend(np.array(g["q"]), np.array(g["keys"]),
                                    np.array(g["values"]), g["scale"])
    np.testing.assert_allclose(probs, g["expected_probs"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out, g["expected_out"], rtol=0, atol=1e-14)
    assert abs(lse - g["expected_lse"]) < 1e-15
    bout, blse = brute.softmax_attend(g["q"], g["keys"], g["values"], g["scale"])
    np.testing.assert_allclose(bout, g["expected_out"], rtol=0, atol=1e-14)
    assert abs(blse - g["expected_lse"]) < 1e-15


def test_golden_causal_prefill(golden_dir):
    g = load_golden(golden_dir, "causal_prefill_closed_form.json")
    q = np.array(g["q"], dtype=np.float32)
    k = np.array(g["k"], dtype=np.float32)
    v = np.array(g["v"], dtype=np.float32)
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    out, lse = oracle.prefill(q, k, v, cu, g["scale"], oracle.F32)
    # inputs are float32 (k = ln 2 rounded), so compare at float32 resolution
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), rtol=0, atol=1e-6)


def test_golden_gqa_group_map(golden_dir):
    g = load_golden(golden_dir, "gqa_group_map.json")
    Hq, Hkv, d, bs = g["num_q_heads"], g["num_kv_heads"], g["head_dim"], g["block_size"]
    kp = np.zeros((1, Hkv, bs, d), dtype=np.float32)
    vp = np.zeros_like(kp)
    vp[0, :, 0, :] = np.array(g["kv_head_values"], dtype=np.float32)
    q = np.ones((1, Hq, d), dtype=np.float32)
    out, _ = oracle.decode(q, kp, vp, np.zeros((1, 1), np.int32), np.array([1], np.int32),
                           bs, g["scale"], oracle.F32)
    np.testing.assert_array_equal(out[0, :, 0], np.array(g["expected_out_per_q_head"]))


def test_golden_lse_merge(golden_dir):
    g = load_golden(golden_dir, "lse_merge_closed_form.json")
    po = np.array(g["part_out"])[None, None]
    pl = np.array(g["part_lse"])[None, None]
    out, lse = oracle.reduce_partitions(po, pl, np.array([g["context_len"]]), g["partition_size"])
    np.testing.assert_allclose(out[0, 0], g["expected_out"], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - g["expected_lse"]) < 1e-15


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_kv_write_untouched_and_skip(dtype):
    rng = np.random.default_rng(7)
    NB, H, bs, d, T = 6, 3, 4, 8, 9
    if dtype == oracle.BF16:
        kp = rng.integers(0, 2 ** 16, (NB, H, bs, d), dtype=np.uint16)
        kn = rng.integers(0, 2 ** 16, (T, H, d), dtype=np.uint16)
    else:
        kp = rand_f32(rng, NB, H, bs, d)
        kn = rand_f32(rng, T, H, d)
    vp, vn = kp[::-1].copy(), kn[::-1].copy()
    slots = rng.permutation(NB * bs)[:T].astype(np.int32)
    slots[[2, 5]] = -1
    kc, vc = oracle.kv_write(kp, vp, kn, vn, slots, bs)
    written = np.zeros((NB, bs), bool)
    for t, s in enumerate(slots):
        if s >= 0:
            blk, off = s // bs, s % bs
            written[blk, off] = True
            assert kc[blk, :, off, :].tobytes() == kn[t].tobytes()
            assert vc[blk, :, off, :].tobytes() == vn[t].tobytes()
    keep = ~written
    assert kc.transpose(0, 2, 1, 3)[keep].tobytes() == kp.transpose(0, 2, 1, 3)[keep].tobytes()
    assert vc.transpose(0, 2, 1, 3)[keep].tobytes() == vp.transpose(0, 2, 1, 3)[keep].tobytes()
    # brute-force spelling gives the same pools
    bk, bv = brute.write_slots(kp.tolist(), vp.tolist(), kn.tolist(), vn.tolist(), slots.tolist(), bs)
    np.testing.assert_array_equal(np.array(bk, dtype=kp.dtype), kc)
    np.testing.assert_array_equal(np.array(bv, dtype=vp.dtype), vc)


# ---------------------------------------------------------------------------
# decode against a library routine on unpaged data
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv,d,bs,lens", [
    (4, 2, 64, 16, (1, 17, 33, 64)),
    (8, 2, 32, 16, (5, 16, 31)),
    (8, 8, 16, 32, (3, 40)),
    (6, 3, 8, 8, (1, 9, 64)),
])
def test_decode_equals_unpaged_sdpa(Hq, Hkv, d, bs, lens):
    rng = np.random.default_rng(11)
    Ks = [rand_f32(rng, n, Hkv, d) for n in lens]
    Vs = [rand_f32(rng, n, Hkv, d) for n in lens]
    q = rand_f32(rng, len(lens), Hq, d)
    kp, vp, tables, ctx = paged_batch(Ks, Vs, bs, rng)
    scale = 1 / math.sqrt(d)
    out, lse = oracle.decode(q, kp, vp, tables, ctx, bs, scale, oracle.F32)
    ref_out, ref_lse = sdpa_decode_reference(q, Ks, Vs, scale)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_decode_bf16_upcast_exact():
    # bf16 inputs are widened exactly: same numbers stored as fp32 give identical results
    rng = np.random.default_rng(3)
    case = wl.make_case(1, dtype=wl.BF16)
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new,
                             case.slot_mapping, case.spec.block_size)
    o1, l1 = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens,
                           case.spec.block_size, case.scale, oracle.BF16)
    as32 = lambda a: wl.bf16_bits_to_f32(a)
    o2, l2 = oracle.decode(as32(case.q), as32(kc), as32(vc), case.block_tables,
                           case.context_lens, case.spec.block_size, case.scale, oracle.F32)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    del rng


# ---------------------------------------------------------------------------
# invariants of the paging model
# ---------------------------------------------------------------------------
def _case1_written():
    case = wl.make_case(1)
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new,
                             case.slot_mapping, case.spec.block_size)
    return case, kc, vc


def test_block_permutation_invariance():
    case, kc, vc = _case1_written()
    rng = np.random.default_rng(5)
    NB = kc.shape[0]
    perm = rng.permutation(NB)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    tables2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    a = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, 16, case.scale, oracle.F32)
    b = oracle.decode(case.q, kc2, vc2, tables2, case.context_lens, 16, case.scale, oracle.F32)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_block_size_invariance():
    rng = np.random.default_rng(9)
    lens = (1, 17, 33, 64, 100)
    Ks = [rand_f32(rng, n, 2, 64) for n in lens]
    Vs = [rand_f32(rng, n, 2, 64) for n in lens]
    q = rand_f32(rng, len(lens), 4, 64)
    res = []
    for bs in (8, 16, 32, 64):
        kp, vp, tables, ctx = paged_batch(Ks, Vs, bs, rng)
        res.append(oracle.decode(q, kp, vp, tables, ctx, bs, 0.125, oracle.F32))
    for o, l in res[1:]:
        np.testing.assert_array_equal(o, res[0][0])
        np.testing.assert_array_equal(l, res[0][1])


def test_gqa_group1_equals_mha():
    case, kc, vc = _case1_written()
    G = case.spec.num_q_heads // case.spec.num_kv_heads
    kc_rep = np.repeat(kc, G, axis=1)
    vc_rep = np.repeat(vc, G, axis=1)
    a = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, 16, case.scale, oracle.F32)
    b = oracle.decode(case.q, kc_rep, vc_rep, case.block_tables, case.context_lens, 16, case.scale, oracle.F32)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_probabilities_sum_to_one_and_constant_v():
    case, kc, vc = _case1_written()
    _, _, probs = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, 16,
                                case.scale, oracle.F32, return_probs=True)
    for p in probs.values():
        assert abs(p.sum() - 1.0) <= 1e-12
        assert (p >= 0).all()
    const = np.float32(0.7421875)
    vconst = np.where(np.isnan(vc), vc, const).astype(np.float32)
    out, _ = oracle.decode(case.q, kc, vconst, case.block_tables, case.context_lens, 16,
                           case.scale, oracle.F32)
    np.testing.assert_allclose(out, const, rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    case, kc, vc = _case1_written()
    b = int(np.argmin(case.context_lens))
    assert case.context_lens[b] == 1
    out, lse = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, 16,
                             case.scale, oracle.F32)
    blk = case.block_tables[b, 0]
    for h in range(case.spec.num_q_heads):
        g = h // 2
        np.testing.assert_array_equal(out[b, h], vc[blk, g, 0].astype(np.float64))
        expect = case.scale * float(np.dot(case.q[b, h].astype(np.float64), kc[blk, g, 0].astype(np.float64)))
        assert abs(lse[b, h] - expect) < 1e-12


@pytest.mark.parametrize("pos", [0, 5, 15, 16, 31, 47, 63])
def test_needle_picks_one_value(pos):
    rng = np.random.default_rng(pos)
    n, Hkv, d, bs = 64, 2, 64, 16
    q = rand_f32(rng, 1, 4, d)
    K = np.zeros((n, Hkv, d), np.float32)
    V = rand_f32(rng, n, Hkv, d)
    for g in range(Hkv):
        qa = q[0, 2 * g]
        K[pos, g] = (200.0 / (0.125 * float(qa @ qa))) * qa
    kp, vp, ids = page_contiguous(K, V, bs, rng)
    out, lse = oracle.decode(q, kp, vp, ids[None], np.array([n], np.int32), bs, 0.125, oracle.F32)
    for h in (0, 2):
        np.testing.assert_allclose(out[0, h], V[pos, h // 2], rtol=1e-80, atol=0)
        assert abs(lse[0, h] - 200.0) < 1e-3


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,over", [
    (1, {}),
    (2, dict(batch=2, ctx_min=1, ctx_max=40, num_q_heads=4, num_kv_heads=2, head_dim=8, max_blocks_per_seq=3)),
    (4, dict(batch=8, ctx_min=32, ctx_max=64, num_q_heads=8, num_kv_heads=2, head_dim=8, block_size=8,
             share_blocks=2, max_blocks_per_seq=8)),
    (5, dict(batch=2, ctx_fixed=(64, 64), num_blocks=12, max_blocks_per_seq=4, head_dim=8,
             num_q_heads=4, num_kv_heads=2)),
])
def test_decode_brute_force_agreement(cfg, over):
    case = wl.make_case(cfg, **over)
    dt = case.spec.dtype
    bs = case.spec.block_size
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    out, lse = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, bs, case.scale, dt)
    bout, blse = brute.paged_decode(oracle.upcast(case.q, dt).tolist(), oracle.upcast(kc, dt).tolist(),
                                    oracle.upcast(vc, dt).tolist(), case.block_tables.tolist(),
                                    case.context_lens.tolist(), bs, case.scale)
    np.testing.assert_allclose(out, np.array(bout), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(blse), rtol=0, atol=1e-12)


def test_prefill_brute_force_agreement():
    case = wl.make_case(3, num_seqs=3, lens_fixed=(1, 7, 20), num_q_heads=4, num_kv_heads=2, head_dim=8)
    dt = case.spec.dtype
    out, lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, dt)
    bout, blse = brute.causal_prefill(oracle.upcast(case.q, dt).tolist(), oracle.upcast(case.k, dt).tolist(),
                                      oracle.upcast(case.v, dt).tolist(), case.cu_seqlens.tolist(), case.scale)
    np.testing.assert_allclose(out, np.array(bout), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(blse), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# split-KV partitions and the merge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("psize", [16, 32, 48, 64, 256])
def test_split_then_merge_equals_unsplit(psize):
    case = wl.make_case(2, batch=5, ctx_min=1, ctx_max=200, num_q_heads=8, num_kv_heads=2,
                        head_dim=16, max_blocks_per_seq=13)
    bs = case.spec.block_size
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    args = (case.q, kc, vc, case.block_tables, case.context_lens, bs, case.scale, wl.BF16)
    full_out, full_lse = oracle.decode(*args)
    P = oracle.num_partitions(case.max_context_len, psize)
    po, pl = oracle.decode_partitions(*args, psize, P)
    # a partition past the end of its sequence carries lse -inf and zero output
    for b in range(case.spec.batch):
        live = -(-int(case.context_lens[b]) // psize)
        assert np.all(np.isneginf(pl[b, :, live:]))
        assert np.all(po[b, :, live:] == 0)
        assert np.all(np.isfinite(pl[b, :, :live]))
    out, lse = oracle.reduce_partitions(po, pl, case.context_lens, psize)
    np.testing.assert_allclose(out, full_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, full_lse, rtol=0, atol=1e-12)


def test_merge_single_partition_is_identity():
    rng = np.random.default_rng(1)
    po = rng.standard_normal((3, 4, 1, 8))
    pl = rng.standard_normal((3, 4, 1))
    out, lse = oracle.reduce_partitions(po, pl, np.array([5, 16, 1]), 16)
    np.testing.assert_array_equal(out, po[:, :, 0])
    np.testing.assert_array_equal(lse, pl[:, :, 0])


def test_merge_ignores_partitions_past_the_end():
    po = np.full((1, 1, 4, 2), 1e30)
    po[0, 0, 0] = [1.0, 2.0]
    pl = np.zeros((1, 1, 4))
    out, lse = oracle.reduce_partitions(po, pl, np.array([10]), 16)
    np.testing.assert_array_equal(out[0, 0], [1.0, 2.0])
    assert lse[0, 0] == 0.0


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def test_prefill_equals_dense_causal_sdpa():
    case = wl.make_case(3, num_seqs=4, lens_fixed=(1, 9, 64, 130), num_q_heads=8, num_kv_heads=2, head_dim=32)
    dt = case.spec.dtype
    out, lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, dt)
    cu = case.cu_seqlens
    for s in range(4):
        a, e = int(cu[s]), int(cu[s + 1])
        Q = torch.from_numpy(oracle.upcast(case.q[a:e], dt)).permute(1, 0, 2)
        K = torch.from_numpy(oracle.upcast(case.k[a:e], dt)).permute(1, 0, 2).repeat_interleave(4, 0)
        V = torch.from_numpy(oracle.upcast(case.v[a:e], dt)).permute(1, 0, 2).repeat_interleave(4, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=True,
                                                                scale=case.scale)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[a:e], ref, rtol=0, atol=1e-12)
        S = (Q @ K.transpose(1, 2)) * case.scale
        S = S.masked_fill(torch.ones(e - a, e - a, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(lse[a:e], torch.logsumexp(S, -1).T.numpy(), rtol=0, atol=1e-12)


def test_prefill_row0_is_v0_and_last_row_matches_decode():
    case = wl.make_case(3, num_seqs=3, lens_fixed=(1, 17, 48), num_q_heads=4, num_kv_heads=2, head_dim=16)
    dt = case.spec.dtype
    out, lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale, dt)
    cu = case.cu_seqlens
    for s in range(3):
        a = int(cu[s])
        for h in range(4):
            np.testing.assert_array_equal(out[a, h], oracle.upcast(case.v[a, h // 2], dt))
            exp = case.scale * float(oracle.upcast(case.q[a, h], dt) @ oracle.upcast(case.k[a, h // 2], dt))
            assert abs(lse[a, h] - exp) < 1e-12
    # cross-path: the last row of each sequence is a decode over the written pool
    pool_k = wl.empty_pool(case.num_blocks, 2, case.spec.block_size, 16, dt)
    pool_v = pool_k.copy()
    kc, vc = oracle.kv_write(pool_k, pool_v, case.k, case.v, case.slot_mapping, case.spec.block_size)
    last = cu[1:] - 1
    dout, dlse = oracle.decode(case.q[last], kc, vc, case.block_tables, np.diff(cu).astype(np.int32),
                               case.spec.block_size, case.scale, dt)
    np.testing.assert_allclose(out[last], dout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[last], dlse, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# paged prefill (a chunk of queries against a cached prefix plus itself)
# ---------------------------------------------------------------------------
def _paged_prefill_inputs(rng, ctxs, chunks, Hq, Hkv, d, bs):
    """Contiguous K/V per sequence paged into one shuffled pool, plus packed q."""
    Ks = [rand_f32(rng, n, Hkv, d) for n in ctxs]
    Vs = [rand_f32(rng, n, Hkv, d) for n in ctxs]
    kp, vp, tables, ctx = paged_batch(Ks, Vs, bs, rng)
    cu = np.zeros(len(chunks) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunks)
    q = rand_f32(rng, int(cu[-1]), Hq, d)
    return Ks, Vs, kp, vp, tables, ctx, cu, q


@pytest.mark.parametrize("ctxs,chunks,bs", [
    ((7, 40, 100), (7, 13, 1), 16),
    ((33, 64, 17), (5, 64, 16), 8),
    ((1, 200), (1, 77), 32),
])
def test_paged_prefill_equals_masked_sdpa(ctxs, chunks, bs):
    # torch SDPA on unpaged K/V with an explicit bottom-right causal mask
    rng = np.random.default_rng(21)
    Hq, Hkv, d = 8, 2, 32
    Ks, Vs, kp, vp, tables, ctx, cu, q = _paged_prefill_inputs(rng, ctxs, chunks, Hq, Hkv, d, bs)
    scale = 0.2
    out, lse = oracle.paged_prefill(q, kp, vp, tables, cu, ctx, bs, scale, oracle.F32)
    for s, (n, lq) in enumerate(zip(ctxs, chunks)):
        a = int(cu[s])
        Q = torch.from_numpy(q[a:a + lq].astype(np.float64)).permute(1, 0, 2)            # [Hq, lq, d]
        K = torch.from_numpy(Ks[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        V = torch.from_numpy(Vs[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        allowed = torch.arange(n)[None, :] <= (n - lq + torch.arange(lq))[:, None]       # [lq, n]
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=allowed,
                                                                scale=scale)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[a:a + lq], ref, rtol=0, atol=1e-12)
        S = ((Q @ K.transpose(1, 2)) * scale).masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(lse[a:a + lq], torch.logsumexp(S, -1).T.numpy(), rtol=0, atol=1e-12)


def test_paged_prefill_special_cases():
    rng = np.random.default_rng(22)
    Hq, Hkv, d, bs = 4, 2, 16, 16
    ctxs = (1, 20, 48)
    # a chunk that is the whole sequence is the plain causal prefill of it
    Ks, Vs, kp, vp, tables, ctx, cu, q = _paged_prefill_inputs(rng, ctxs, ctxs, Hq, Hkv, d, bs)
    out, lse = oracle.paged_prefill(q, kp, vp, tables, cu, ctx, bs, 0.25, oracle.F32)
    pout, plse = oracle.prefill(q, np.concatenate(Ks), np.concatenate(Vs), cu, 0.25, oracle.F32)
    np.testing.assert_allclose(out, pout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, plse, rtol=0, atol=1e-12)
    # a one-row chunk is a decode of that row over the whole cache
    cu1 = np.arange(len(ctxs) + 1, dtype=np.int32)
    q1 = rand_f32(rng, len(ctxs), Hq, d)
    out1, lse1 = oracle.paged_prefill(q1, kp, vp, tables, cu1, ctx, bs, 0.25, oracle.F32)
    dout, dlse = oracle.decode(q1, kp, vp, tables, ctx, bs, 0.25, oracle.F32)
    np.testing.assert_allclose(out1, dout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, dlse, rtol=0, atol=1e-12)
    # more rows than cached positions is an error
    with pytest.raises(ValueError):
        oracle.paged_prefill(q[:3], kp, vp, tables, np.array([0, 2, 2, 3], np.int32),
                             np.array([1, 20, 48], np.int32), bs, 0.25, oracle.F32)


def test_paged_prefill_brute_force_and_permutation():
    case = wl.make_case(6, num_seqs=3, prefix_fixed=(0, 5, 21), chunk_fixed=(3, 1, 11),
                        num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=8)
    dt = case.spec.dtype
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, 8)
    out, lse = oracle.paged_prefill(case.q, kc, vc, case.block_tables, case.cu_seqlens_q,
                                    case.context_lens, 8, case.scale, dt)
    up = lambda x: oracle.upcast(x, dt).tolist()
    bout, blse = brute.paged_prefill(up(case.q), up(kc), up(vc), case.block_tables.tolist(),
                                     case.cu_seqlens_q.tolist(), case.context_lens.tolist(), 8, case.scale)
    np.testing.assert_allclose(out, np.array(bout), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(blse), rtol=0, atol=1e-12)
    # moving every physical block elsewhere (tables follow) changes nothing
    perm = np.random.default_rng(5).permutation(kc.shape[0])
    kp = np.empty_like(kc)
    vp = np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc
    tables = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.paged_prefill(case.q, kp, vp, tables, case.cu_seqlens_q, case.context_lens, 8,
                                      case.scale, dt)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)


# ---------------------------------------------------------------------------
# sliding window (keys max(0, p - W + 1) .. p)
# ---------------------------------------------------------------------------
def page_window_mask(rows, keys, window, offset=0):
    """The page's construction, written out: for row i (at position offset + i)
    the keys start = max(0, pos - window + 1) .. pos are open, the rest closed."""
    allowed = torch.zeros((rows, keys), dtype=torch.bool)
    for i in range(rows):
        pos = offset + i
        start = max(0, pos - window + 1)
        allowed[i, start:pos + 1] = True
    return allowed


def free_before_window(tables, first_keys, block_size):
    """Tables whose entries for blocks ending at or before each sequence's
    first visible key are -1 (blocks a server may have freed)."""
    ft = tables.copy()
    for b, k0 in enumerate(first_keys):
        ft[b, :int(k0) // block_size] = -1
    return ft


@pytest.mark.parametrize("window", [1, 5, 64, 1000])
def test_window_prefill_and_paged_prefill_equal_masked_sdpa(window):
    rng = np.random.default_rng(31)
    Hq, Hkv, d, bs = 4, 2, 16, 8
    ctxs, chunks = (9, 70, 130), (9, 20, 77)
    Ks, Vs, kp, vp, tables, ctx, cu, q = _paged_prefill_inputs(rng, ctxs, chunks, Hq, Hkv, d, bs)
    pout, plse = oracle.paged_prefill(q, kp, vp, tables, cu, ctx, bs, 0.3, oracle.F32, window=window)
    # the full-sequence chunk (first sequence) also goes through the varlen prefill
    fout, flse = oracle.prefill(q[:9], Ks[0], Vs[0], np.array([0, 9], np.int32), 0.3, oracle.F32, window=window)
    np.testing.assert_allclose(fout, pout[:9], rtol=0, atol=1e-12)
    np.testing.assert_allclose(flse, plse[:9], rtol=0, atol=1e-12)
    for s, (n, lq) in enumerate(zip(ctxs, chunks)):
        a = int(cu[s])
        Q = torch.from_numpy(q[a:a + lq].astype(np.float64)).permute(1, 0, 2)
        K = torch.from_numpy(Ks[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
        V = torch.from_numpy(Vs[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
        allowed = page_window_mask(lq, n, window, offset=n - lq)
        ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=allowed,
                                                                scale=0.3)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(pout[a:a + lq], ref, rtol=0, atol=1e-12)
        S = ((Q @ K.transpose(1, 2)) * 0.3).masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(plse[a:a + lq], torch.logsumexp(S, -1).T.numpy(), rtol=0, atol=1e-12)
    # blocks before the first row's window may be freed
    ft = free_before_window(tables, [max(0, n - lq - window + 1) for n, lq in zip(ctxs, chunks)], bs)
    fo, fl = oracle.paged_prefill(q, kp, vp, ft, cu, ctx, bs, 0.3, oracle.F32, window=window)
    np.testing.assert_array_equal(fo, pout)
    np.testing.assert_array_equal(fl, plse)


@pytest.mark.parametrize("window", [1, 7, 40, 500])
def test_window_decode_equals_masked_sdpa_and_split_merge(window):
    rng = np.random.default_rng(32)
    Hq, Hkv, d, bs, lens = 4, 2, 16, 16, (1, 17, 33, 130)
    Ks = [rand_f32(rng, n, Hkv, d) for n in lens]
    Vs = [rand_f32(rng, n, Hkv, d) for n in lens]
    q = rand_f32(rng, len(lens), Hq, d)
    kp, vp, tables, ctx = paged_batch(Ks, Vs, bs, rng)
    out, lse = oracle.decode(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, window=window)
    for b, n in enumerate(lens):
        allowed = page_window_mask(1, n, window, offset=n - 1)[0]
        Kw, Vw = Ks[b][allowed.numpy()], Vs[b][allowed.numpy()]
        ref_out, ref_lse = sdpa_decode_reference(q[b:b + 1], [Kw], [Vw], 0.25)
        np.testing.assert_allclose(out[b], ref_out[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_lse[0], rtol=0, atol=1e-12)
    for ps in (16, 32):
        po, pl = oracle.decode_partitions(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, ps, window=window)
        mo, ml = oracle.reduce_partitions(po, pl, ctx, ps)
        np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)
        # the window-aware merge never reads the partitions before the window
        first = [max(0, n - window) // ps for n in lens]
        for b, f in enumerate(first):
            po[b, :, :f], pl[b, :, :f] = np.nan, np.nan
        mo, ml = oracle.reduce_partitions(po, pl, ctx, ps, window=window)
        np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)
    # blocks wholly before the window may be freed: their table entries are
    # never looked up
    ft = free_before_window(tables, [max(0, n - window) for n in lens], bs)
    fo, fl = oracle.decode(q, kp, vp, ft, ctx, bs, 0.25, oracle.F32, window=window)
    np.testing.assert_array_equal(fo, out)
    np.testing.assert_array_equal(fl, lse)
    # a window of one key returns the newest value; a window past the start changes nothing
    o1, _ = oracle.decode(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, window=1)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(o1[b], np.repeat(Vs[b][n - 1], 2, axis=0).astype(np.float64))
    ow, lw = oracle.decode(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32, window=130)
    on, ln = oracle.decode(q, kp, vp, tables, ctx, bs, 0.25, oracle.F32)
    np.testing.assert_array_equal(ow, on)
    np.testing.assert_array_equal(lw, ln)


# ---------------------------------------------------------------------------
# the generator itself
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,over", [
    (1, {}),
    (2, dict(batch=6, ctx_min=1, ctx_max=100, max_blocks_per_seq=7)),
    (4, dict(batch=16, ctx_min=512, ctx_max=700, max_blocks_per_seq=22)),
])
def test_generator_layout(cfg, over):
    a = wl.make_case(cfg, **over)
    b = wl.make_case(cfg, **over)
    assert a.q.tobytes() == b.q.tobytes() and a.k_cache.tobytes() == b.k_cache.tobytes()
    bs = a.spec.block_size
    NB = a.num_blocks
    ids = a.block_tables[a.block_tables >= 0]
    assert ids.min() >= 0 and ids.max() < NB
    if not a.spec.share_group:
        assert len(np.unique(ids)) == len(ids)
    if a.slot_mapping.size:
        assert len(np.unique(a.slot_mapping)) == a.slot_mapping.size
        assert a.slot_mapping.max() < NB * bs
    # history positions finite; position ctx-1 (pending write) and unused slots NaN
    kf = wl.bf16_bits_to_f32(a.k_cache) if a.spec.dtype == wl.BF16 else a.k_cache
    used = np.zeros((NB, bs), bool)
    for bi in range(a.spec.batch):
        hist = int(a.context_lens[bi]) - (1 if a.spec.write_new_token else 0)
        for p in range(hist):
            blk = a.block_tables[bi, p // bs]
            used[blk, p % bs] = True
            assert np.isfinite(kf[blk, :, p % bs]).all()
    assert np.isnan(kf.transpose(0, 2, 1, 3)[~used]).all()


@pytest.mark.parametrize("cfg,over", [
    (1, {}),
    (2, dict(batch=8, ctx_min=100, ctx_max=700, max_blocks_per_seq=44)),
    (4, dict(batch=8, ctx_min=600, ctx_max=900, max_blocks_per_seq=29)),
])
def test_needle_on_workloads(cfg, over):
    """The needle inputs the GPU tests use select exactly one value row in the oracle."""
    from tests.gpu_util import needle_case, needle_targets, storage_to_f64
    rng = np.random.default_rng(77)
    for r in (0, 5, 63):
        case = wl.make_case(cfg, **over)
        targets = needle_targets(case, r, rng)
        case = needle_case(case, targets)
        bs = case.spec.block_size
        kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
        out, lse = oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, bs, case.scale,
                                 case.spec.dtype)
        G = case.spec.num_q_heads // case.spec.num_kv_heads
        for b, t in enumerate(targets):
            v = storage_to_f64(vc[case.block_tables[b, t // bs], :, t % bs, :])
            for h in range(case.spec.num_q_heads):
                np.testing.assert_allclose(out[b, h], v[h // G], rtol=1e-60, atol=0)
            assert np.all(np.abs(lse[b] - 200.0) < 2.0)
