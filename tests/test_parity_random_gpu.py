"""Seeded random-shape GPU parity against the fp64 CPU oracle, through the C ABI.

Every case draws its own shape from a fixed seed: dtype (bf16 / f32), head_dim
(64 / 128), GQA group (1, 2, 4, 8), KV heads, block size (8 .. 64), batch,
context or prompt lengths (empty sequences, single tokens, lengths either side
of a tile edge, a few hundred), split-KV partition size (0 = single pass),
sliding window (0 = none, else 1 .. 300 keys, with blocks wholly before it
freed for some decodes), the softmax scale, the slack between the host-side
bounds (max_context_len, max_seqlen) and the real maxima, the value
distribution, and whether the step's cache write runs as its own launch or
inside the decode (append) and whether bf16 / head_dim 128 is forced onto the
vector kernels.  Outputs start as NaN so that a row the kernels skip fails.
Pools written on the GPU are compared bit for bit with the oracle's write.

The draws are host logic: a CPU test checks that they are valid and that
together they reach every value listed above.
A wide regime (up to 8 KV heads, 24 sequences, contexts to 8,192, prompts to
1,500, cached prefixes to 3,000, windows to 3,000) adds a few draws of each
kind; PA_PARITY_DRAWS=k multiplies every count for a longer sweep.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import assert_parity, to_dev, to_host_bits, to_host_f64

# PA_PARITY_DRAWS=k multiplies every count below (a longer sweep); the wide
# regime (contexts to 8192, batches to 24, windows to 3000) has few draws by
# default since its oracle side takes about a second a case.
SCALE = max(1, int(os.environ.get("PA_PARITY_DRAWS", "1")))
N_DECODE, N_PREFILL, N_PAGED, N_FP8 = 200 * SCALE, 100 * SCALE, 100 * SCALE, 60 * SCALE
W_DECODE, W_PREFILL, W_PAGED, W_FP8 = 16 * SCALE, 10 * SCALE, 8 * SCALE, 6 * SCALE

NARROW = dict(seed=0, hkv=5, batch=9, ctx=1200, window=301, parts=(1, 2, 4, 8, 16), fp8_parts=(1, 2, 4, 8),
              seqs=7, prompt=400, prefix=400, chunk=250)
WIDE = dict(seed=10000, hkv=9, batch=25, ctx=8192, window=3001, parts=(1, 4, 16, 32), fp8_parts=(1, 4, 16),
            seqs=25, prompt=1500, prefix=3000, chunk=800)


def _lengths(rng, n, hi, allow_zero=True):
    """n lengths mixing 0, 1, tile edges +-1 and uniform draws up to hi."""
    out = []
    for _ in range(n):
        r = rng.random()
        if r < 0.1 and allow_zero:
            out.append(0)
        elif r < 0.2:
            out.append(1)
        elif r < 0.45:
            edge = int(rng.choice([16, 32, 64, 128, 256]))
            out.append(min(hi, max(1, edge + int(rng.integers(-1, 2)))))
        else:
            out.append(int(rng.integers(1, hi + 1)))
    return out


def _scale(rng, d):
    return float(np.float32(rng.uniform(0.5, 2.0) / math.sqrt(d)))


def _window(rng, hi=301):
    return 0 if rng.random() < 0.5 else int(rng.choice([1, 2, int(rng.integers(3, hi))]))


def decode_draw(i, rg=NARROW):
    rng = np.random.default_rng(7100 + rg["seed"] + i)
    dtype = wl.BF16 if rng.random() < 0.6 else wl.F32
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, rg["hkv"]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, rg["batch"]))
    ctx = _lengths(rng, B, rg["ctx"])
    if max(ctx) == 0:
        ctx[0] = int(rng.integers(1, 300))
    nblk = max(-(-c // bs) for c in ctx)
    mbps = nblk + int(rng.integers(0, 4))
    maxctx = int(rng.integers(max(ctx), mbps * bs + 1))
    window = _window(rng, rg["window"])
    return dict(
        seed=9100 + rg["seed"] + i, dtype=dtype, head_dim=d, num_q_heads=G * Hkv, num_kv_heads=Hkv, block_size=bs,
        batch=B, ctx_fixed=tuple(ctx), max_blocks_per_seq=mbps, max_context_len=maxctx,
        partition_size=0 if rng.random() < 0.35 else bs * int(rng.choice(rg["parts"])),
        window=window, free_before_window=bool(window and rng.random() < 0.5),
        v_dist=str(rng.choice(["normal", "uniform"])), scale=_scale(rng, d),
        append=bool(rng.random() < 0.3), vector=bool(dtype == wl.BF16 and d == 128 and rng.random() < 0.3),
        pool_factor=float(rng.choice([1.0, 1.25, 2.0])))


def fp8_draw(i, rg=NARROW):
    rng = np.random.default_rng(7400 + rg["seed"] + i)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, rg["hkv"]))
    bs = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, rg["batch"]))
    ctx = _lengths(rng, B, rg["ctx"])
    if max(ctx) == 0:
        ctx[0] = int(rng.integers(1, 300))
    nblk = max(-(-c // bs) for c in ctx)
    mbps = nblk + int(rng.integers(0, 4))
    window = _window(rng, rg["window"])
    return dict(
        seed=9400 + rg["seed"] + i, num_q_heads=G * Hkv, num_kv_heads=Hkv, block_size=bs, batch=B, ctx_fixed=tuple(ctx),
        max_blocks_per_seq=mbps, max_context_len=int(rng.integers(max(ctx), mbps * bs + 1)),
        partition_size=0 if rng.random() < 0.35 else bs * int(rng.choice(rg["fp8_parts"])),
        window=window, free_before_window=bool(window and rng.random() < 0.5),
        k_scale=float(rng.uniform(2.0, 8.0) / 448.0), v_scale=float(rng.uniform(2.0, 8.0) / 448.0),
        v_dist=str(rng.choice(["normal", "uniform"])), scale=_scale(rng, 128))


def prefill_draw(i, rg=NARROW):
    rng = np.random.default_rng(7200 + rg["seed"] + i)
    dtype = wl.BF16 if rng.random() < 0.6 else wl.F32
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, rg["hkv"]))
    S = int(rng.integers(1, rg["seqs"]))
    lens = _lengths(rng, S, rg["prompt"])
    if max(lens) == 0:
        lens[0] = int(rng.integers(1, 200))
    T = sum(lens)
    return dict(
        seed=9200 + rg["seed"] + i, dtype=dtype, head_dim=d, num_q_heads=G * Hkv, num_kv_heads=Hkv, num_seqs=S,
        lens_fixed=tuple(lens), max_seqlen=int(rng.integers(max(lens), T + 1)), window=_window(rng, rg["window"]),
        scale=_scale(rng, d), vector=bool(dtype == wl.BF16 and d == 128 and rng.random() < 0.3))


def paged_draw(i, rg=NARROW):
    rng = np.random.default_rng(7300 + rg["seed"] + i)
    dtype = wl.BF16 if rng.random() < 0.6 else wl.F32
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, rg["hkv"]))
    bs = int(rng.choice([8, 16, 32, 64]))
    S = int(rng.integers(1, rg["seqs"]))
    prefix = _lengths(rng, S, rg["prefix"])
    chunk = _lengths(rng, S, rg["chunk"])
    if max(chunk) == 0:
        chunk[0] = int(rng.integers(1, 100))
    T = sum(chunk)
    ctx = [p + c for p, c in zip(prefix, chunk)]
    mbps = max(1, max(-(-c // bs) for c in ctx))
    return dict(
        seed=9300 + rg["seed"] + i, dtype=dtype, head_dim=d, num_q_heads=G * Hkv, num_kv_heads=Hkv, block_size=bs,
        num_seqs=S, prefix_fixed=tuple(prefix), chunk_fixed=tuple(chunk),
        max_seqlen_q=int(rng.integers(max(chunk), T + 1)),
        max_context_len=int(rng.integers(max(ctx), mbps * bs + 1)), window=_window(rng, rg["window"]),
        scale=_scale(rng, d), vector=bool(dtype == wl.BF16 and d == 128 and rng.random() < 0.3))


def _cases(tag, n_narrow, n_wide):
    return ([pytest.param(NARROW, i, id=f"{tag}{i:02d}") for i in range(n_narrow)] +
            [pytest.param(WIDE, i, id=f"wide_{tag}{i:02d}") for i in range(n_wide)])

_HOST_KEYS = ("seed", "max_context_len", "max_seqlen", "max_seqlen_q", "scale", "append", "vector")


def _spec_args(draw):
    return {k: v for k, v in draw.items() if k not in _HOST_KEYS}


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


# ---------------------------------------------------------------------------
# host logic: the draws are valid and reach every listed value (CPU)
# ---------------------------------------------------------------------------
def test_random_draws_are_valid_and_cover_the_space():
    dec = [decode_draw(i) for i in range(N_DECODE)]
    pre = [prefill_draw(i) for i in range(N_PREFILL)]
    pag = [paged_draw(i) for i in range(N_PAGED)]
    f8 = [fp8_draw(i) for i in range(N_FP8)]
    for c in dec + f8:
        assert c["num_q_heads"] // c["num_kv_heads"] in (1, 2, 4, 8)
        assert max(c["ctx_fixed"]) <= c["max_context_len"] <= c["max_blocks_per_seq"] * c["block_size"]
        assert c["partition_size"] % c["block_size"] == 0
    for c in pre:
        assert max(c["lens_fixed"]) <= c["max_seqlen"] <= sum(c["lens_fixed"])
    for c in pag:
        assert max(c["chunk_fixed"]) <= c["max_seqlen_q"] <= sum(c["chunk_fixed"])
    every = dec + pre + pag
    assert {c["dtype"] for c in every} == {wl.BF16, wl.F32}
    assert {c["head_dim"] for c in every} == {64, 128}
    assert {c["num_q_heads"] // c["num_kv_heads"] for c in dec} == {1, 2, 4, 8}
    assert {c["num_q_heads"] // c["num_kv_heads"] for c in pre} == {1, 2, 4, 8}
    assert {c["num_q_heads"] // c["num_kv_heads"] for c in pag} == {1, 2, 4, 8}
    assert {c["block_size"] for c in dec} == {8, 16, 32, 64}
    assert {c["block_size"] for c in pag} == {8, 16, 32, 64}
    assert {c["block_size"] for c in f8} == {16, 32, 64}
    for group in (dec, f8):
        assert any(c["partition_size"] == 0 for c in group) and any(c["partition_size"] for c in group)
        assert any(c["free_before_window"] for c in group)
        assert any(c["max_context_len"] > max(c["ctx_fixed"]) for c in group)
    for group in (dec, pre, pag, f8):
        assert any(c["window"] == 0 for c in group) and any(c["window"] > 0 for c in group)
    assert any(c["window"] == 1 for c in dec + pre + pag + f8)
    assert any(0 in c["ctx_fixed"] for c in dec) and any(1 in c["ctx_fixed"] for c in dec)
    assert any(0 in c["lens_fixed"] for c in pre) and any(1 in c["lens_fixed"] for c in pre)
    assert any(0 in c["prefix_fixed"] for c in pag) and any(0 in c["chunk_fixed"] for c in pag)
    assert any(c["append"] for c in dec) and any(c["vector"] for c in dec)
    assert any(c["vector"] for c in pre) and any(c["vector"] for c in pag)
    assert any(c["append"] and c["partition_size"] and c["window"] for c in dec)
    assert any(c["max_seqlen"] > max(c["lens_fixed"]) for c in pre)
    assert any(c["max_seqlen_q"] > max(c["chunk_fixed"]) for c in pag)
    # the wide regime reaches what the narrow one does not
    wd = [decode_draw(i, WIDE) for i in range(W_DECODE)] + [fp8_draw(i, WIDE) for i in range(W_FP8)]
    wp = [prefill_draw(i, WIDE) for i in range(W_PREFILL)]
    wg = [paged_draw(i, WIDE) for i in range(W_PAGED)]
    for c in wd:
        assert max(c["ctx_fixed"]) <= c["max_context_len"] <= c["max_blocks_per_seq"] * c["block_size"]
    assert max(max(c["ctx_fixed"]) for c in wd) > 4096 and max(c["window"] for c in wd) > 1000
    assert max(c["num_kv_heads"] for c in wd + wp + wg) > 4 and max(c["batch"] for c in wd) > 8
    assert max(max(c["lens_fixed"]) for c in wp) > 400 and max(max(c["prefix_fixed"]) for c in wg) > 400


# ---------------------------------------------------------------------------
# decode (+ reduce), bf16 / f32 pools
# ---------------------------------------------------------------------------
@pytest.mark.gpu
@pytest.mark.parametrize("rg,i", _cases("decode", N_DECODE, W_DECODE))
def test_random_decode(rg, i):
    draw = decode_draw(i, rg)
    print("decode", draw, flush=True)
    case = wl.make_case(2, seed=draw["seed"], name="random_decode", **_spec_args(draw))
    sp, bs, ps, window = case.spec, case.spec.block_size, draw["partition_size"], draw["window"]
    maxctx, scale = draw["max_context_len"], draw["scale"]
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    kn = vn = None
    if draw["append"]:
        kn, vn = to_dev(case.k_new), to_dev(case.v_new)
    elif case.slot_mapping.size:
        ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    B, Hq, d = case.q.shape
    ops.set_force_vector_path(draw["vector"])
    try:
        out, lse = _nan((B, Hq, d), q.dtype), _nan((B, Hq), torch.float32)
        if ps:
            P = ops.num_partitions(maxctx, ps)
            po, pl = _nan((B, Hq, P, d), torch.float32), _nan((B, Hq, P), torch.float32)
            ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, scale, ps, part_out=po, part_lse=pl,
                                       window=window, k_new=kn, v_new=vn)
            ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, out=out, lse=lse, window=window)
        else:
            ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, scale, out=out, lse=lse, window=window,
                                       k_new=kn, v_new=vn)
        torch.cuda.synchronize()
    finally:
        ops.set_force_vector_path(False)
    okc, ovc = case.k_cache, case.v_cache
    if case.slot_mapping.size:
        okc, ovc = oracle.kv_write(okc, ovc, case.k_new, case.v_new, case.slot_mapping, bs)
    np.testing.assert_array_equal(to_host_bits(kc), okc)
    np.testing.assert_array_equal(to_host_bits(vc), ovc)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, scale,
                                     sp.dtype, window=window)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, sp.dtype, f"decode draw {i}")


# ---------------------------------------------------------------------------
# decode over E4M3 pools (bf16 queries, head_dim 128)
# ---------------------------------------------------------------------------
@pytest.mark.gpu
@pytest.mark.parametrize("rg,i", _cases("fp8_", N_FP8, W_FP8))
def test_random_decode_fp8(rg, i):
    draw = fp8_draw(i, rg)
    print("fp8 decode", draw, flush=True)
    case = wl.make_case(8, seed=draw["seed"], name="random_fp8", **_spec_args(draw))
    bs, ps, window, maxctx, scale = (case.spec.block_size, draw["partition_size"], draw["window"],
                                     draw["max_context_len"], draw["scale"])
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    if case.slot_mapping.size:
        ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping),
                           k_scale=ks, v_scale=vs)
    q, bt, cl = to_dev(case.q), to_dev(case.block_tables), to_dev(case.context_lens)
    B, Hq, d = case.q.shape
    out, lse = _nan((B, Hq, d), q.dtype), _nan((B, Hq), torch.float32)
    if ps:
        P = ops.num_partitions(maxctx, ps)
        po, pl = _nan((B, Hq, P, d), torch.float32), _nan((B, Hq, P), torch.float32)
        ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, scale, ps, part_out=po, part_lse=pl,
                                   window=window, k_scale=ks, v_scale=vs)
        ops.paged_attention_reduce(po, pl, cl, ps, out_dtype=q.dtype, out=out, lse=lse, window=window)
    else:
        ops.paged_attention_decode(q, kc, vc, bt, cl, maxctx, scale, out=out, lse=lse, window=window,
                                   k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    okc, ovc = case.k_cache, case.v_cache
    if case.slot_mapping.size:
        okc, ovc = oracle.kv_write_fp8(okc, ovc, case.k_new, case.v_new, case.slot_mapping, bs,
                                       case.spec.dtype, case.k_scale, case.v_scale)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
    ref_out, ref_lse = oracle.decode(case.q, okc, ovc, case.block_tables, case.context_lens, bs, scale,
                                     case.spec.dtype, window=window, kv_dtype=oracle.E4M3,
                                     k_scale=case.k_scale, v_scale=case.v_scale)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"fp8 draw {i}")


# ---------------------------------------------------------------------------
# varlen causal prefill
# ---------------------------------------------------------------------------
@pytest.mark.gpu
@pytest.mark.parametrize("rg,i", _cases("prefill", N_PREFILL, W_PREFILL))
def test_random_prefill(rg, i):
    draw = prefill_draw(i, rg)
    print("prefill", draw, flush=True)
    window, scale = draw["window"], draw["scale"]
    case = wl.make_case(3, seed=draw["seed"], name="random_prefill",
                        **{k: v for k, v in _spec_args(draw).items() if k != "window"})
    q, k, v, cu = to_dev(case.q), to_dev(case.k), to_dev(case.v), to_dev(case.cu_seqlens)
    T, Hq, d = case.q.shape
    out, lse = _nan((T, Hq, d), q.dtype), _nan((T, Hq), torch.float32)
    ops.set_force_vector_path(draw["vector"])
    try:
        ops.varlen_causal_prefill(q, k, v, cu, draw["max_seqlen"], scale, out=out, lse=lse, window=window)
        torch.cuda.synchronize()
    finally:
        ops.set_force_vector_path(False)
    ref_out, ref_lse = oracle.prefill(case.q, case.k, case.v, case.cu_seqlens, scale, case.spec.dtype,
                                      window=window)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"prefill draw {i}")


# ---------------------------------------------------------------------------
# paged (chunked / prefix-cached) prefill
# ---------------------------------------------------------------------------
@pytest.mark.gpu
@pytest.mark.parametrize("rg,i", _cases("paged", N_PAGED, W_PAGED))
def test_random_paged_prefill(rg, i):
    draw = paged_draw(i, rg)
    print("paged prefill", draw, flush=True)
    window, scale = draw["window"], draw["scale"]
    case = wl.make_case(6, seed=draw["seed"], name="random_paged",
                        **{k: v for k, v in _spec_args(draw).items() if k != "window"})
    bs = case.spec.block_size
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    if case.slot_mapping.size:
        ops.paged_kv_write(to_dev(case.k_new), to_dev(case.v_new), kc, vc, to_dev(case.slot_mapping))
    q = to_dev(case.q)
    T, Hq, d = case.q.shape
    out, lse = _nan((T, Hq, d), q.dtype), _nan((T, Hq), torch.float32)
    ops.set_force_vector_path(draw["vector"])
    try:
        ops.paged_prefill(q, kc, vc, to_dev(case.block_tables), to_dev(case.cu_seqlens_q),
                          to_dev(case.context_lens), draw["max_seqlen_q"], draw["max_context_len"], scale,
                          out=out, lse=lse, window=window)
        torch.cuda.synchronize()
    finally:
        ops.set_force_vector_path(False)
    okc, ovc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    np.testing.assert_array_equal(to_host_bits(kc), okc)
    np.testing.assert_array_equal(to_host_bits(vc), ovc)
    ref_out, ref_lse = oracle.paged_prefill(case.q, okc, ovc, case.block_tables, case.cu_seqlens_q,
                                            case.context_lens, bs, scale, case.spec.dtype, window=window)
    assert_parity(to_host_f64(out), to_host_f64(lse), ref_out, ref_lse, case.spec.dtype, f"paged draw {i}")
