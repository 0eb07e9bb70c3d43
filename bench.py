"""Benchmark: attention over a paged KV cache on one MI355X.

One step = the decode hot path on the Llama-3-8B-shaped workload (64
sequences, 32 query / 8 KV heads, head_dim 128, 16-token blocks, contexts
uniform in [128, 2048], shuffled pool 1.25x the need): the cache write of the
64 new tokens folded into the split-KV decode (paged_attention_decode_append,
1024-token partitions), then paged_attention_reduce.  The headline value is
KV-cache bytes streamed per second (sum of context lengths x 8 KV heads x
(K + V) x 128 x 2 bytes per step).  Beside it: the same step as three
launches (paged_kv_write first), both steps captured in a HIP graph, the
decode kernel alone at other partition sizes, and the paged stream probe
(paged_kv_stream_read: the same units and tiles read with no attention, the
ceiling of decode's access pattern) with torch's copy and sum.

Inputs are resident in HBM before timing.  Independent copies of the pools,
tables and queries are rotated so the 256 MB Infinity Cache cannot serve one
step's KV from the previous step.  Secondary figures, each with its own
roofline: the varlen causal prefill on the Llama-3-8B varlen workload (16
sequences, lengths uniform in [64, 2048]; TFLOP/s over unmasked query-key
pairs), the prompt cache write and the fused RoPE cache write of its rows,
the chunked paged prefill (16 sequences, cached prefix 0..3072, chunk
128..1024); under a 2048-key sliding window, the split decode of 64 sequences
of 1024..16384 positions (GB/s over the window's KV bytes) and the chunked
paged prefill; the decode over an E4M3 cache (512-token partitions) and its
history write; the Llama-2-70B prefix-shared decode (256 sequences, GB/s over
unique KV bytes) and the long-context split decode (4 x 131072 positions).
The fp64 oracle is timed on the host cores beside the decode, the prefill and
the two large decode workloads.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode KV GB/s (% HBM peak); varlen prefill TFLOP/s; Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
DECODE_SOURCES = ("attention_paged_kv_write_amd/csrc/decode.hip",
                  "attention_paged_kv_write_amd/csrc/units.h",
                  "attention_paged_kv_write_amd/csrc/common.h",
                  "attention_paged_kv_write_amd/csrc/kernels.h")
PREFILL_SOURCES = ("attention_paged_kv_write_amd/csrc/prefill.hip",
                   "attention_paged_kv_write_amd/csrc/common.h",
                   "attention_paged_kv_write_amd/csrc/kernels.h")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_llama3_8b.txt")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_llama3_8b.txt")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_fp8_llama3_8b.txt")
PAGED_PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_paged_prefill_llama3_8b.txt")
WINDOW_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_window_llama3_8b.txt")
ROPE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rope_kv_write_llama3_8b.txt")
KV_WRITE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_kv_write_prompt_llama3_8b.txt")
C4_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_llama2_70b_prefix.txt")
C5_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_long_context.txt")
KV_WRITE_SOURCES = ("attention_paged_kv_write_amd/csrc/kv_write.hip",
                    "attention_paged_kv_write_amd/csrc/common.h",
                    "attention_paged_kv_write_amd/csrc/kernels.h")
ROPE_SOURCES = ("attention_paged_kv_write_amd/csrc/rope.hip",
                "attention_paged_kv_write_amd/csrc/common.h",
                "attention_paged_kv_write_amd/csrc/kernels.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path, sources):
    """HBM bytes per launch of a kernel from committed rocprofv3 counters, if
    the kernel's sources are unchanged since they were taken; else None."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest(sources):
        return None
    return t.get("traffic_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return 1


def host_note():
    return f"host cpu_count={os.cpu_count()} affinity={len(os.sched_getaffinity(0))}"


def prefill_cpu_baseline(pc, seconds):
    """The fp64 oracle's varlen prefill on whole sequences of the same
    workload, in order, until `seconds` have passed: TFLOP/s over the same
    algorithmic FLOP count as the GPU figure."""
    import oracle
    lens = np.diff(pc.cu_seqlens).astype(np.int64)
    t0 = time.perf_counter()
    done, fl = 0, 0.0
    while time.perf_counter() - t0 < seconds and done < len(lens):
        oracle.prefill(pc.q, pc.k, pc.v, pc.cu_seqlens, pc.scale, pc.spec.dtype, seqs=[done])
        fl += 4.0 * pc.spec.head_dim * pc.spec.num_q_heads * float(lens[done] * (lens[done] + 1) // 2)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"fp64 NumPy oracle prefill of the first {done} of {len(lens)} sequences "
                      f"({int(lens[:done].sum())} rows, all {pc.spec.num_q_heads} heads) in {dt:.2f} s; "
                      f"BLAS threads {blas_threads()}, {host_note()}"}


def decode_cpu_baseline(case, seconds, unique_bytes_per_kv_byte=1.0, pools=None, window=0, kv8=False, seqs=None):
    """The fp64 oracle's decode of whole sequences of the same workload, in
    order (cycling over the first `seqs`), until `seconds` have passed: GB/s of
    the KV the queries see (the last `window` positions under a window; one
    byte per element for an E4M3 pool).  `pools`: the (k, v) pools to read
    when not the case's own (written on the host by the oracle)."""
    import oracle
    spec = case.spec
    B, Hkv, d = spec.batch, spec.num_kv_heads, spec.head_dim
    kc, vc = pools if pools is not None else (case.k_cache, case.v_cache)
    fp8 = dict(kv_dtype=oracle.E4M3, k_scale=case.k_scale, v_scale=case.v_scale) if kv8 else {}
    per_pos = Hkv * 2 * d * (1 if kv8 else 2)
    nseq = min(B, seqs) if seqs else B
    t0 = time.perf_counter()
    n, nbytes = 0, 0
    while time.perf_counter() - t0 < seconds:
        b = n % nseq
        oracle.decode(case.q[b:b + 1], kc, vc, case.block_tables[b:b + 1], case.context_lens[b:b + 1],
                      spec.block_size, case.scale, spec.dtype, window=window, **fp8)
        n += 1
        ctx = int(case.context_lens[b])
        nbytes += (min(ctx, window) if window else ctx) * per_pos
    dt = time.perf_counter() - t0
    return {"value": round(nbytes * unique_bytes_per_kv_byte / dt / 1e9, 4), "unit": "GB/s",
            "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"fp64 NumPy oracle decode of {n} sequences in order ({nbytes / 1e6:.1f} MB of KV) "
                      f"in {dt:.2f} s; BLAS threads {blas_threads()}, {host_note()}"}


def window_cpu_baseline(case, window, seconds):
    """The oracle's sliding-window decode of the window workload (its new
    tokens written on the host first)."""
    import oracle
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping,
                             case.spec.block_size)
    return decode_cpu_baseline(case, seconds, pools=(kc, vc), window=window)


def fp8_cpu_baseline(case, seconds, nseq=12):
    """The oracle's decode over an E4M3 pool: the first `nseq` sequences'
    history written by the oracle's FP8 write (not timed), then decoded in
    order until `seconds` have passed."""
    import oracle
    tok = int(case.context_lens[:nseq].sum())   # the workload lists each sequence's positions in order
    kc, vc = oracle.kv_write_fp8(case.k_cache, case.v_cache, case.k_new[:tok], case.v_new[:tok],
                                 case.slot_mapping[:tok], case.spec.block_size, case.spec.dtype, case.k_scale,
                                 case.v_scale)
    r = decode_cpu_baseline(case, seconds, pools=(kc, vc), kv8=True, seqs=nseq)
    r["sample"] += f" (the first {nseq} sequences, their E4M3 history written by the oracle beforehand)"
    return r


def paged_prefill_cpu_baseline(case, seconds):
    """The oracle's paged prefill of whole sequences in order (the chunks'
    K/V written on the host first): TFLOP/s over the GPU figure's count."""
    import oracle
    bs = case.spec.block_size
    kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
    lq = np.diff(case.cu_seqlens_q).astype(np.int64)
    pre = case.context_lens.astype(np.int64) - lq
    t0 = time.perf_counter()
    done, fl = 0, 0.0
    while time.perf_counter() - t0 < seconds and done < len(lq):
        oracle.paged_prefill(case.q, kc, vc, case.block_tables, case.cu_seqlens_q, case.context_lens, bs, case.scale,
                             case.spec.dtype, seqs=[done])
        fl += 4.0 * case.spec.head_dim * case.spec.num_q_heads * float(lq[done] * pre[done] + lq[done] * (lq[done] + 1) // 2)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"fp64 NumPy oracle paged prefill of the first {done} of {len(lq)} sequences "
                      f"({int(lq[:done].sum())} query rows, all {case.spec.num_q_heads} heads) in {dt:.2f} s; "
                      f"BLAS threads {blas_threads()}, {host_note()}"}


def rope_cpu_baseline(pc, positions, rot_dim, base, bytes_per_token):
    """The oracle's fused RoPE cache write over the prompt rows, once: GB/s of
    the same algorithmic bytes per token as the GPU figure."""
    from oracle import rope
    from attention_paged_kv_write_amd import workloads as wl
    spec = pc.spec
    pool = wl.empty_pool(pc.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim, spec.dtype)
    t0 = time.perf_counter()
    rope.rope_kv_write(pc.q, pc.k, pc.v, pool, pool.copy(), pc.slot_mapping, positions, spec.block_size, rot_dim,
                       base, spec.dtype)
    dt = time.perf_counter() - t0
    T = pc.total_tokens
    return {"value": round(bytes_per_token * T / dt / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle RoPE cache write of all {T} prompt rows once in {dt:.2f} s; "
                      f"BLAS threads {blas_threads()}, {host_note()}"}


def timed_groups(torch, stream, fn, n_items, n_groups, group=10):
    """Per-launch ms of fn(i) over n_groups groups of `group` back-to-back
    launches (i rotating over n_items input copies), HIP events recorded on
    the launch stream around each group."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_groups)]
    torch.cuda.synchronize()
    for gi in range(n_groups):
        evs[gi][0].record(stream)
        for k in range(group):
            fn((gi * group + k) % n_items)
        evs[gi][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / group for a, b in evs]


def graph_ms(torch, stream, fn, n_items, reps):
    """ms per fn(i) when the n_items calls are captured once in a HIP graph
    and the graph is replayed `reps` times (no host launch cost); None if the
    capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_items):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_items):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (reps * n_items)
        del g
        return ms
    except Exception as e:  # pragma: no cover - depends on the runtime
        log(f"graph capture failed: {e}")
        return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition-size", type=int, default=1024,
                    help="split-KV partition of the headline decode step (the fastest of those timed in "
                         "roofline.partition_size_variants on MI355X)")
    ap.add_argument("--fp8-partition-size", type=int, default=512,
                    help="split-KV partition of the E4M3 decode (256 and 512 within 1%% on MI355X; 512 leaves "
                         "the merge half the partials)")
    ap.add_argument("--copies", type=int, default=3, help="independent input copies rotated per step")
    ap.add_argument("--prefill-iters", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-window", action="store_true", help="skip the sliding-window figures")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache figures")
    ap.add_argument("--no-c4", action="store_true", help="skip the Llama-2-70B prefix-sharing decode figures")
    ap.add_argument("--no-c5", action="store_true", help="skip the long-context split-KV decode figures")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-captured step timings")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 5 times (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from attention_paged_kv_write_amd import ops
    from attention_paged_kv_write_amd import workloads as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    ops.load_library()
    build_id = ops.check_build_id()   # the .so that runs is the one built from these sources
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": 5}))
        return

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    # ------------------------------------------------------------------ decode
    t0 = time.perf_counter()
    case = wl.make_case(2)
    spec = case.spec
    log(f"decode workload generated in {time.perf_counter() - t0:.1f}s: "
        f"NB={case.num_blocks} sum(ctx)={int(case.context_lens.sum())}")
    B, Hq, Hkv, d, bs = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    ps = args.partition_size
    maxctx = case.max_context_len
    P = ops.num_partitions(maxctx, ps)
    copies = []
    for _ in range(max(1, args.copies)):
        copies.append(dict(q=up(case.q), kc=up(case.k_cache), vc=up(case.v_cache),
                           bt=up(case.block_tables), cl=up(case.context_lens),
                           kn=up(case.k_new), vn=up(case.v_new), slots=up(case.slot_mapping),
                           po=torch.empty((B, Hq, P, d), dtype=torch.float32, device=dev),
                           pl=torch.empty((B, Hq, P), dtype=torch.float32, device=dev),
                           out=torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev),
                           lse=torch.empty((B, Hq), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()

    # one decode step: the new tokens' cache write folded into the split decode
    # (paged_attention_decode_append), then the log-sum-exp merge
    def step(c):
        ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], maxctx, case.scale, ps,
                                   part_out=c["po"], part_lse=c["pl"], k_new=c["kn"], v_new=c["vn"])
        ops.paged_attention_reduce(c["po"], c["pl"], c["cl"], ps, out=c["out"], lse=c["lse"])

    # the same step as three launches (paged_kv_write first), for reference
    def step_separate(c):
        ops.paged_kv_write(c["kn"], c["vn"], c["kc"], c["vc"], c["slots"])
        ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], maxctx, case.scale, ps,
                                   part_out=c["po"], part_lse=c["pl"])
        ops.paged_attention_reduce(c["po"], c["pl"], c["cl"], ps, out=c["out"], lse=c["lse"])

    for i in range(args.warmup):
        step(copies[i % len(copies)])
    torch.cuda.synchronize()
    log("decode warmup done")

    # timed region: K whole steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(copies[i % len(copies)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    log(f"decode steps timed: {ms_per_step * 1e3:.1f} us/step")
    torch.cuda.synchronize()
    t_sep = time.perf_counter()
    for i in range(args.steps):
        step_separate(copies[i % len(copies)])
    torch.cuda.synchronize()
    sep_ms = (time.perf_counter() - t_sep) * 1e3 / args.steps
    log(f"same step as three launches: {sep_ms * 1e3:.1f} us/step")

    # The decode kernel alone: back-to-back launches (rotating the copies) between
    # HIP events recorded on the stream the kernel runs on, in groups of 10, so
    # a launch's dispatch overlaps the previous kernel as in the timed steps.
    def decode_only(c):
        ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], maxctx, case.scale, ps,
                                   part_out=c["po"], part_lse=c["pl"])
    group = 10
    n_groups = max(1, args.steps // group)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_groups)]
    torch.cuda.synchronize()
    for gi in range(n_groups):
        evs[gi][0].record(stream)
        for k in range(group):
            decode_only(copies[(gi * group + k) % len(copies)])
        evs[gi][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) / group for a, b in evs]
    dec_avg_ms = float(np.mean(dec_ms))

    kv_bytes = int(case.context_lens.astype(np.int64).sum()) * Hkv * 2 * d * 2
    value_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved_gbs = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)
    roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "kernel": "decode_mfma_kernel<G=4,BS=16,W=1> (paged_attention_decode)",
                "kernel_avg_us": round(dec_avg_ms * 1e3, 2),
                "kernel_median_us": round(float(np.median(dec_ms)) * 1e3, 2),
                "kernel_p10_us": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                "kernel_p90_us": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                "timing": "HIP events on the launch stream around groups of 10 back-to-back launches",
                "algorithmic_bytes_per_launch": kv_bytes}
    log(f"decode kernel avg {dec_avg_ms * 1e3:.1f} us -> {achieved_gbs:.0f} GB/s")

    g2 = g3 = None
    stream_ceiling = None
    try:
        # Both steps again with their launches captured in a HIP graph (one capture
        # holds one step per input copy), so the figure is GPU time, not Python.
        graph_reps = max(1, args.steps // len(copies))
        if not args.no_graph:
            g2 = graph_ms(torch, stream, lambda i: step(copies[i]), len(copies), graph_reps)
            g3 = graph_ms(torch, stream, lambda i: step_separate(copies[i]), len(copies), graph_reps)
        log(f"graph-captured step: {g2 * 1e3 if g2 else float('nan'):.1f} us (two launches), "
            f"{g3 * 1e3 if g3 else float('nan'):.1f} us (three launches)")

        # The same decode kernel at other partition sizes (0 = one pass per
        # (sequence, KV head) writing out/lse directly, no reduce needed).
        variants = {}
        for vps in sorted({0, 256, 512, 768, 1024} - {ps}):
            vP = ops.num_partitions(maxctx, vps) if vps else 1
            vbuf = [dict(po=torch.empty((B, Hq, vP, d), dtype=torch.float32, device=dev),
                         pl=torch.empty((B, Hq, vP), dtype=torch.float32, device=dev)) if vps else None
                    for _ in copies]

            def vdecode(i, vps=vps, vbuf=vbuf):
                c = copies[i]
                if vps:
                    ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], maxctx, case.scale, vps,
                                               part_out=vbuf[i]["po"], part_lse=vbuf[i]["pl"])
                else:
                    ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], maxctx, case.scale,
                                               out=c["out"], lse=c["lse"])
            for i in range(len(copies)):
                vdecode(i)
            vms = float(np.mean(timed_groups(torch, stream, vdecode, len(copies), n_groups)))
            variants[str(vps)] = {"kernel_avg_us": round(vms * 1e3, 2),
                                  "gbs": round(kv_bytes / (vms * 1e-3) / 1e9, 1)}
            del vbuf
        roofline["partition_size_variants"] = variants
        log("decode kernel by partition size: " +
            ", ".join(f"{k}: {v['kernel_avg_us']} us" for k, v in variants.items()))

        # Paged stream probe: the decode's work units and tiles read with no
        # attention (paged_kv_stream_read), LDS-DMA rings of 2 (the decode
        # kernel's), 3 and 4 slots, and register loads 4 tiles at a time.
        sums = [torch.empty((B, Hkv, P), dtype=torch.int32, device=dev) for _ in copies]
        probe = {}
        for mode, depth, name in ((ops.PA_STREAM_LDS_DMA, 2, "lds_dma_ring_2"), (ops.PA_STREAM_LDS_DMA, 3, "lds_dma_ring_3"),
                                  (ops.PA_STREAM_LDS_DMA, 4, "lds_dma_ring_4"), (ops.PA_STREAM_REGISTERS, 4, "registers_4")):
            def sread(i, mode=mode, depth=depth):
                c = copies[i]
                ops.paged_kv_stream_read(c["kc"], c["vc"], c["bt"], c["cl"], maxctx, ps, mode, depth, checksums=sums[i])
            for i in range(len(copies)):
                sread(i)
            sms = float(np.mean(timed_groups(torch, stream, sread, len(copies), n_groups)))
            probe[name] = {"kernel_avg_us": round(sms * 1e3, 2), "gbs": round(kv_bytes / (sms * 1e-3) / 1e9, 1)}
        best_probe = max(v["gbs"] for v in probe.values())
        log("paged stream probe: " + ", ".join(f"{k}: {v['gbs']} GB/s" for k, v in probe.items()))
        del sums
        # Plain read ceiling beside it: the same pools read front to back, every
        # byte once (pa_stream_read_contiguous: 2048 waves, 4 loads in flight per
        # lane), the six pools of the three copies rotated.
        pools = [c[k] for c in copies for k in ("kc", "vc")]
        pool_bytes = pools[0].numel() * pools[0].element_size()
        csum = torch.empty((2048,), dtype=torch.int32, device=dev)

        def cread(i):
            ops.stream_read_contiguous(pools[i], waves=2048, depth=4, checksums=csum)
        for i in range(len(pools)):
            cread(i)
        cms = float(np.mean(timed_groups(torch, stream, cread, len(pools), n_groups)))
        contiguous = {"bytes_per_launch": pool_bytes, "kernel_avg_us": round(cms * 1e3, 2),
                      "gbs": round(pool_bytes / (cms * 1e-3) / 1e9, 1)}
        del pools
        del copies
        torch.cuda.empty_cache()

        # Practical HBM ceiling on this machine: a plain 1 GiB device copy (read + write).
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ca.record(stream)
        for _ in range(5):
            dst.copy_(src)
        cb.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * nb * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
        src.zero_()
        f32 = src.view(torch.float32)
        f32.sum()
        ca.record(stream)
        for _ in range(5):
            f32.sum()
        cb.record(stream)
        torch.cuda.synchronize()
        read_gbs = nb * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
        csum = torch.empty((2048,), dtype=torch.int32, device=dev)
        ops.stream_read_contiguous(src, waves=2048, depth=4, checksums=csum)
        ca.record(stream)
        for _ in range(5):
            ops.stream_read_contiguous(src, waves=2048, depth=4, checksums=csum)
        cb.record(stream)
        torch.cuda.synchronize()
        contiguous["gbs_1gib"] = round(nb * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9, 1)
        stream_ceiling = {"kind": "paged stream probe on the decode workload's own pools, tables and work units "
                                  "(paged_kv_stream_read, KV bytes per launch / launch time); the plain read of the "
                                  "same pools front to back and of 1 GiB (pa_stream_read_contiguous); torch on 1 GiB: "
                                  "device copy (read + write bytes) and fp32 sum (read bytes)",
                          "paged_stream": probe,
                          "contiguous_read": contiguous,
                          "copy_gbs": round(copy_gbs, 1), "read_gbs": round(read_gbs, 1),
                          "frac_of_peak": round(max(copy_gbs, read_gbs, best_probe, contiguous["gbs"],
                                                    contiguous["gbs_1gib"]) / HBM_PEAK_GBS, 4),
                          "decode_over_best_paged_stream": round(achieved_gbs / best_probe, 4),
                          "decode_over_contiguous_read": round(achieved_gbs / contiguous["gbs"], 4)}
        log(f"contiguous read: pools {contiguous['gbs']} GB/s, 1 GiB {contiguous['gbs_1gib']} GB/s; "
            f"device copy {copy_gbs:.0f} GB/s, sum {read_gbs:.0f} GB/s")
        del src, dst
        torch.cuda.empty_cache()
    except Exception as e:  # a failing secondary figure must not cost the headline line
        log(f"graph / partition variants / stream ceiling failed: {e!r}")
        stream_ceiling = {"error": repr(e)}
        torch.cuda.empty_cache()

    # ----------------------------------------------------------------- prefill
    prefill = None
    try:
        if not args.no_prefill:
            t0 = time.perf_counter()
            pc = wl.make_case(3)
            log(f"prefill workload generated in {time.perf_counter() - t0:.1f}s: T={pc.total_tokens}")
            lens = np.diff(pc.cu_seqlens).astype(np.int64)
            flops = 4.0 * pc.spec.head_dim * pc.spec.num_q_heads * float((lens * (lens + 1) // 2).sum())
            # q, k, v read once; out and lse written once
            T_, Hq_, Hkv_, d_ = pc.total_tokens, pc.spec.num_q_heads, pc.spec.num_kv_heads, pc.spec.head_dim
            io_bytes = T_ * (2 * Hq_ + 2 * Hkv_) * d_ * 2 + T_ * Hq_ * 4
            # two copies of q, k, v (2 x 211 MB) alternate, so one launch's inputs
            # are not in the 256 MB Infinity Cache from the launch before
            pcu = up(pc.cu_seqlens)
            pcopies = [dict(q=up(pc.q), k=up(pc.k), v=up(pc.v)) for _ in range(2)]
            for c in pcopies:
                c["out"] = torch.empty_like(c["q"])
                c["lse"] = torch.empty((pc.total_tokens, pc.spec.num_q_heads), dtype=torch.float32, device=dev)
            pq, pk, pv = pcopies[0]["q"], pcopies[0]["k"], pcopies[0]["v"]

            def pfill(i):
                c = pcopies[i]
                ops.varlen_causal_prefill(c["q"], c["k"], c["v"], pcu, pc.max_seqlen, pc.scale, out=c["out"],
                                          lse=c["lse"])
            for i in range(3):
                pfill(i % 2)
            p_ms = timed_groups(torch, stream, pfill, 2, max(1, args.prefill_iters // 5), group=5)
            pms = float(np.mean(p_ms))
            tflops = flops / (pms * 1e-3) / 1e12
            # paged write-through of the prompt K/V: four copies of the source rows
            # (4 x 70 MB) and two pools alternate; HIP events around groups of 10
            # back-to-back writes
            pools = [(torch.empty((pc.num_blocks, pc.spec.num_kv_heads, pc.spec.block_size, pc.spec.head_dim),
                                  dtype=torch.bfloat16, device=dev),
                      torch.empty((pc.num_blocks, pc.spec.num_kv_heads, pc.spec.block_size, pc.spec.head_dim),
                                  dtype=torch.bfloat16, device=dev)) for _ in range(2)]
            pool, pool_v = pools[0]
            wsrc = [(pcopies[0]["k"], pcopies[0]["v"]), (pcopies[1]["k"], pcopies[1]["v"]),
                    (up(pc.k), up(pc.v)), (up(pc.k), up(pc.v))]
            slots = up(pc.slot_mapping)

            def pwrite(i):
                ops.paged_kv_write(wsrc[i][0], wsrc[i][1], pools[i % 2][0], pools[i % 2][1], slots)
            for i in range(4):
                pwrite(i)
            wms = float(np.mean(timed_groups(torch, stream, pwrite, 4, 2)))
            wbytes = 2 * 2 * pc.total_tokens * pc.spec.num_kv_heads * pc.spec.head_dim * 2  # read + write, K and V
            # RoPE fused into the prompt's cache write (row positions 0 .. L-1 of each
            # sequence, base 10000): q and k rotated in place, rotated k and v into
            # the pool; on two copies of q, k, v (every call turns q and k again)
            cu_h = pc.cu_seqlens.astype(np.int64)
            rpos = torch.from_numpy(np.concatenate([np.arange(cu_h[i + 1] - cu_h[i]) for i in range(len(cu_h) - 1)])
                                    .astype(np.int32)).to(dev)
            rtab = ops.rope_cos_sin_cache(pc.max_seqlen, d_, 10000.0)
            rope_bytes = (2 * T_ * Hq_ * d_ * 2 + 3 * T_ * Hkv_ * d_ * 2 + 2 * T_ * Hkv_ * d_ * 2
                          + T_ * d_ * 4 + T_ * 8)

            def rwrite(i):
                c = pcopies[i]
                ops.paged_kv_write_rope(c["q"], c["k"], c["v"], pools[i][0], pools[i][1], slots, rpos, rtab)
            for i in range(2):
                rwrite(i)
            rms = float(np.mean(timed_groups(torch, stream, rwrite, 2, 2)))
            rgbs = rope_bytes / (rms * 1e-3) / 1e9
            rope_write = {"workload": pc.spec.name + " prompt rows", "rot_dim": d_, "base": 10000.0,
                          "kernel_avg_us": round(rms * 1e3, 1),
                          "roofline": {"bound": "hbm", "achieved": round(rgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(rgbs / HBM_PEAK_GBS, 4),
                                       "traffic": measured_traffic(ROPE_TRAFFIC_FILE, ROPE_SOURCES),
                                       "kernel": "rope_kv_write_kernel<bf16> (paged_kv_write_rope)",
                                       "algorithmic_bytes_per_launch": rope_bytes}}
            log(f"fused rope + kv write {rms * 1e3:.1f} us -> {rgbs:.0f} GB/s")
            prefill = {"workload": pc.spec.name, "total_tokens": pc.total_tokens,
                       "kernel_avg_us": round(pms * 1e3, 1), "tflops": round(tflops, 1),
                       "kernel_median_us": round(float(np.median(p_ms)) * 1e3, 1),
                       "kernel_p10_us": round(float(np.percentile(p_ms, 10)) * 1e3, 1),
                       "kernel_p90_us": round(float(np.percentile(p_ms, 90)) * 1e3, 1),
                       "input_copies": 2,
                       "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                                    "traffic": measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SOURCES),
                                    "kernel": "prefill_mfma_kernel<NW=4> (varlen_causal_prefill)",
                                    "algorithmic_flops_per_launch": flops,
                                    "algorithmic_bytes_per_launch": io_bytes},
                       "tokens_per_s": round(pc.total_tokens / (pms * 1e-3), 1),
                       "kv_write": {"kernel_avg_us": round(wms * 1e3, 1),
                                    "gbs": round(wbytes / (wms * 1e-3) / 1e9, 1),
                                    "traffic": measured_traffic(KV_WRITE_TRAFFIC_FILE, KV_WRITE_SOURCES),
                                    "algorithmic_bytes_per_launch": wbytes,
                                    "input_copies": "4 source copies, 2 pools"},
                       "rope_kv_write": rope_write}
            log(f"prefill {pms * 1e3:.1f} us -> {tflops:.1f} TFLOP/s; prompt kv write {wms * 1e3:.1f} us")
            if not args.no_cpu_baseline:
                prefill["cpu_baseline"] = prefill_cpu_baseline(pc, args.cpu_seconds)
                log(f"prefill cpu baseline {prefill['cpu_baseline']['value']} TFLOP/s")
                try:
                    rope_write["cpu_baseline"] = rope_cpu_baseline(pc, rpos.cpu().numpy(), d_, 10000.0,
                                                                   rope_bytes / T_)
                    log(f"rope write cpu baseline {rope_write['cpu_baseline']['value']} GB/s")
                except Exception as e:  # a baseline must not cost the GPU figures
                    log(f"rope cpu baseline failed: {e!r}")
            del pq, pk, pv, pool, pool_v, pcopies, pools, wsrc
            torch.cuda.empty_cache()

            # chunked prefill against a cached prefix (workload 6): the chunk's K/V are
            # written into the pool first (untimed), then paged_prefill is timed
            cc = wl.make_case(6)
            lq = np.diff(cc.cu_seqlens_q).astype(np.int64)
            pre = cc.context_lens.astype(np.int64) - lq
            cflops = 4.0 * cc.spec.head_dim * cc.spec.num_q_heads * float((lq * pre + lq * (lq + 1) // 2).sum())
            ckc, cvc = up(cc.k_cache), up(cc.v_cache)
            ops.paged_kv_write(up(cc.k_new), up(cc.v_new), ckc, cvc, up(cc.slot_mapping))
            cq, cbt, ccu, ccl = up(cc.q), up(cc.block_tables), up(cc.cu_seqlens_q), up(cc.context_lens)
            cout = torch.empty_like(cq)
            clse = torch.empty((cc.total_q, cc.spec.num_q_heads), dtype=torch.float32, device=dev)

            def chunked():
                ops.paged_prefill(cq, ckc, cvc, cbt, ccu, ccl, cc.max_seqlen_q, cc.max_context_len, cc.scale,
                                  out=cout, lse=clse)
            for _ in range(3):
                chunked()
            torch.cuda.synchronize()
            pa_, pb_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            pa_.record(stream)
            for _ in range(args.prefill_iters):
                chunked()
            pb_.record(stream)
            torch.cuda.synchronize()
            cms = pa_.elapsed_time(pb_) / args.prefill_iters
            ctf = cflops / (cms * 1e-3) / 1e12
            paged_prefill = {"workload": cc.spec.name, "query_rows": cc.total_q,
                             "cached_positions": int(cc.context_lens.sum()),
                             "kernel_avg_us": round(cms * 1e3, 1), "tflops": round(ctf, 1),
                             "roofline": {"bound": "mfma", "achieved": round(ctf, 1), "peak": BF16_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": round(ctf / BF16_PEAK_TFLOPS, 4),
                                          "traffic": measured_traffic(PAGED_PREFILL_TRAFFIC_FILE, PREFILL_SOURCES),
                                          "kernel": "prefill_mfma_kernel<NW=4, paged> (paged_prefill)",
                                          "algorithmic_flops_per_launch": cflops},
                             "tokens_per_s": round(cc.total_q / (cms * 1e-3), 1)}
            prefill["paged_prefill"] = paged_prefill
            log(f"paged prefill {cms * 1e3:.1f} us -> {ctf:.1f} TFLOP/s")
            if not args.no_cpu_baseline:
                try:
                    paged_prefill["cpu_baseline"] = paged_prefill_cpu_baseline(cc, min(args.cpu_seconds, 5.0))
                    log(f"paged prefill cpu baseline {paged_prefill['cpu_baseline']['value']} TFLOP/s")
                except Exception as e:
                    log(f"paged prefill cpu baseline failed: {e!r}")

            del ckc, cvc, cq, cout
            torch.cuda.empty_cache()

            # Length sweep: 16 sequences of L tokens each, the same heads and head
            # size, iid standard-normal values rounded to bf16 drawn on the device
            # (a timing study: the distribution of the workload above, not its draws).
            gen = torch.Generator(device=dev)
            gen.manual_seed(1013)

            def draw(shape):
                return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            sweep = {}
            for L in (256, 1024, 2048, 4096, 8192):
                Ts = 16 * L
                sq, sk, sv = draw((Ts, Hq_, d_)), draw((Ts, Hkv_, d_)), draw((Ts, Hkv_, d_))
                scu = torch.arange(0, Ts + 1, L, dtype=torch.int32, device=dev)
                so = torch.empty_like(sq)
                sl = torch.empty((Ts, Hq_), dtype=torch.float32, device=dev)

                def sfill():
                    ops.varlen_causal_prefill(sq, sk, sv, scu, L, pc.scale, out=so, lse=sl)
                for _ in range(2):
                    sfill()
                n_it = max(3, 8192 // L)
                torch.cuda.synchronize()
                sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                sa.record(stream)
                for _ in range(n_it):
                    sfill()
                sb.record(stream)
                torch.cuda.synchronize()
                sms = sa.elapsed_time(sb) / n_it
                sfl = 4.0 * d_ * Hq_ * 16 * L * (L + 1) / 2
                stf = sfl / (sms * 1e-3) / 1e12
                sweep[str(L)] = {"kernel_avg_us": round(sms * 1e3, 1), "tflops": round(stf, 1),
                                 "frac": round(stf / BF16_PEAK_TFLOPS, 4)}
                del sq, sk, sv, so, sl
            torch.cuda.empty_cache()
            prefill["length_sweep"] = {"num_seqs": 16, "values": "iid standard normal, bf16, drawn on the device",
                                       "by_length": sweep}
            log("prefill length sweep (TFLOP/s): " + ", ".join(f"{k}: {v['tflops']}" for k, v in sweep.items()))

            # The workload's own lengths at Llama-3-8B's heads per GPU under 4- and
            # 8-way tensor parallelism (H_q 8 with H_kv 2 or 1): fewer head columns
            # than XCDs, so the XCDs share each column.
            cu_d = torch.from_numpy(pc.cu_seqlens).to(dev)
            lens_h = np.diff(pc.cu_seqlens).astype(np.int64)
            few = {}
            for hq, hkv in ((8, 2), (8, 1)):
                fq, fk, fv = draw((T_, hq, d_)), draw((T_, hkv, d_)), draw((T_, hkv, d_))
                fo = torch.empty_like(fq)
                fl = torch.empty((T_, hq), dtype=torch.float32, device=dev)

                def ffill():
                    ops.varlen_causal_prefill(fq, fk, fv, cu_d, pc.max_seqlen, pc.scale, out=fo, lse=fl)
                for _ in range(2):
                    ffill()
                torch.cuda.synchronize()
                sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                sa.record(stream)
                for _ in range(10):
                    ffill()
                sb.record(stream)
                torch.cuda.synchronize()
                fms = sa.elapsed_time(sb) / 10
                ftf = 4.0 * d_ * hq * float((lens_h * (lens_h + 1) // 2).sum()) / (fms * 1e-3) / 1e12
                few[f"hq{hq}_hkv{hkv}"] = {"kernel_avg_us": round(fms * 1e3, 1), "tflops": round(ftf, 1),
                                           "frac": round(ftf / BF16_PEAK_TFLOPS, 4)}
                del fq, fk, fv, fo, fl
            torch.cuda.empty_cache()
            prefill["few_kv_heads"] = {"lengths": pc.spec.name + " (same cu_seqlens)",
                                       "values": "iid standard normal, bf16, drawn on the device", "by_heads": few}
            log("prefill, few KV heads (TFLOP/s): " + ", ".join(f"{k}: {v['tflops']}" for k, v in few.items()))

            # The rate the matrix cores sustain on this machine for a plain bf16 GEMM
            # (torch.matmul, 8192^3): the clock under dense matrix work sits well
            # below the 2.4 GHz the 2.5 PFLOP/s peak assumes, so this is the
            # practical ceiling the attention kernel is also measured against.
            ga, gb = draw((8192, 8192)), draw((8192, 8192))
            for _ in range(3):
                gc = ga @ gb
            torch.cuda.synchronize()
            sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            sa.record(stream)
            for _ in range(10):
                gc = ga @ gb
            sb.record(stream)
            torch.cuda.synchronize()
            gtf = 2.0 * 8192 ** 3 / (sa.elapsed_time(sb) / 10 * 1e-3) / 1e12
            prefill["gemm_reference"] = {"op": "torch.matmul bf16 8192 x 8192 x 8192", "tflops": round(gtf, 1),
                                         "frac_of_peak": round(gtf / BF16_PEAK_TFLOPS, 4),
                                         "prefill_over_gemm": round(tflops / gtf, 4),
                                         "length_8192_over_gemm": round(sweep["8192"]["tflops"] / gtf, 4)}
            log(f"bf16 GEMM reference {gtf:.0f} TFLOP/s")
            del ga, gb, gc
            torch.cuda.empty_cache()
    except Exception as e:  # a failing secondary figure must not cost the headline line
        log(f"prefill section failed: {e!r}")
        prefill = {"error": repr(e)}
        torch.cuda.empty_cache()

    # ---------------------------------------------------------- sliding window
    window = None
    try:
        if not args.no_window:
            t0 = time.perf_counter()
            wc = wl.make_case(7)
            W, wps = wc.spec.window, wc.spec.partition_size
            wB, wHq, wHkv, wd = wc.spec.batch, wc.spec.num_q_heads, wc.spec.num_kv_heads, wc.spec.head_dim
            log(f"window workload generated in {time.perf_counter() - t0:.1f}s: NB={wc.num_blocks}")
            # algorithmic bytes: K and V of the visible keys, min(ctx, W) per sequence
            wvis = np.minimum(wc.context_lens.astype(np.int64), W)
            wbytes = int(wvis.sum()) * wHkv * 2 * wd * 2
            wP = ops.num_partitions(wc.max_context_len, wps)
            wcopies = []
            for _ in range(2):   # two pool copies: the window's KV of one launch exceeds the Infinity Cache anyway
                c = dict(q=up(wc.q), kc=up(wc.k_cache), vc=up(wc.v_cache), bt=up(wc.block_tables),
                         cl=up(wc.context_lens),
                         po=torch.empty((wB, wHq, wP, wd), dtype=torch.float32, device=dev),
                         pl=torch.empty((wB, wHq, wP), dtype=torch.float32, device=dev),
                         out=torch.empty((wB, wHq, wd), dtype=torch.bfloat16, device=dev),
                         lse=torch.empty((wB, wHq), dtype=torch.float32, device=dev))
                ops.paged_kv_write(up(wc.k_new), up(wc.v_new), c["kc"], c["vc"], up(wc.slot_mapping))
                wcopies.append(c)

            def wdecode(c):
                ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], wc.max_context_len, wc.scale,
                                           wps, part_out=c["po"], part_lse=c["pl"], window=W)

            def wstep(c):
                wdecode(c)
                ops.paged_attention_reduce(c["po"], c["pl"], c["cl"], wps, out=c["out"], lse=c["lse"], window=W)

            def timed(fn, n_groups):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(n_groups)]
                torch.cuda.synchronize()
                for gi in range(n_groups):
                    evs[gi][0].record(stream)
                    for k in range(group):
                        fn(wcopies[(gi * group + k) % len(wcopies)])
                    evs[gi][1].record(stream)
                torch.cuda.synchronize()
                return [a.elapsed_time(b) / group for a, b in evs]
            for i in range(10):
                wstep(wcopies[i % 2])
            wg = max(1, args.steps // group)
            wdec_ms = timed(wdecode, wg)
            wstep_ms = timed(wstep, wg)
            wavg = float(np.mean(wdec_ms))
            wgbs = wbytes / (wavg * 1e-3) / 1e9
            window = {"workload": wc.spec.name, "window": W, "partition_size": wps,
                      "sum_context": int(wc.context_lens.sum()), "visible_keys": int(wvis.sum()),
                      "kv_bytes_per_step": wbytes,
                      "step_us": round(float(np.mean(wstep_ms)) * 1e3, 2),
                      "step_gbs": round(wbytes / (float(np.mean(wstep_ms)) * 1e-3) / 1e9, 1),
                      "roofline": {"bound": "hbm", "achieved": round(wgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(wgbs / HBM_PEAK_GBS, 4),
                                   "traffic": measured_traffic(WINDOW_TRAFFIC_FILE, DECODE_SOURCES),
                                   "kernel": "decode_mfma_kernel<G=4,BS=16,W=1> (paged_attention_decode_window)",
                                   "kernel_avg_us": round(wavg * 1e3, 2),
                                   "timing": "HIP events on the launch stream around groups of 10 back-to-back launches",
                                   "algorithmic_bytes_per_launch": wbytes},
                      "decode_tokens_per_s": round(wB / (float(np.mean(wstep_ms)) * 1e-3), 1),
                      "paged_prefill": None}
            log(f"window decode kernel {wavg * 1e3:.1f} us -> {wgbs:.0f} GB/s; step {np.mean(wstep_ms) * 1e3:.1f} us")
            if not args.no_cpu_baseline:
                try:
                    window["cpu_baseline"] = window_cpu_baseline(wc, W, min(args.cpu_seconds, 5.0))
                    log(f"window decode cpu baseline {window['cpu_baseline']['value']} GB/s")
                except Exception as e:
                    log(f"window cpu baseline failed: {e!r}")
            del wcopies
            torch.cuda.empty_cache()

            # chunked prefill (workload 6) under the same 2048-key window: the row at
            # position p sees min(p + 1, 2048) keys (runs with the window figures,
            # whatever --no-prefill says)
            if True:
                cc = wl.make_case(6)
                lq = np.diff(cc.cu_seqlens_q).astype(np.int64)
                pre = cc.context_lens.astype(np.int64) - lq
                cflops = 4.0 * cc.spec.head_dim * cc.spec.num_q_heads * float((lq * pre + lq * (lq + 1) // 2).sum())
                PW = W
                vis = np.concatenate([np.minimum(np.arange(p0, p0 + n) + 1, PW) for p0, n in zip(pre, lq)])
                wflops = 4.0 * cc.spec.head_dim * cc.spec.num_q_heads * float(vis.sum())
                ckc, cvc = up(cc.k_cache), up(cc.v_cache)
                ops.paged_kv_write(up(cc.k_new), up(cc.v_new), ckc, cvc, up(cc.slot_mapping))
                cq, cbt, ccu, ccl = up(cc.q), up(cc.block_tables), up(cc.cu_seqlens_q), up(cc.context_lens)
                cout = torch.empty_like(cq)
                clse = torch.empty((cc.total_q, cc.spec.num_q_heads), dtype=torch.float32, device=dev)

                def chunked_w():
                    ops.paged_prefill(cq, ckc, cvc, cbt, ccu, ccl, cc.max_seqlen_q, cc.max_context_len, cc.scale,
                                      out=cout, lse=clse, window=PW)
                for _ in range(3):
                    chunked_w()
                torch.cuda.synchronize()
                pa_, pb_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                pa_.record(stream)
                for _ in range(args.prefill_iters):
                    chunked_w()
                pb_.record(stream)
                torch.cuda.synchronize()
                wpms = pa_.elapsed_time(pb_) / args.prefill_iters
                wtf = wflops / (wpms * 1e-3) / 1e12
                window_prefill = {"workload": cc.spec.name, "window": PW, "kernel_avg_us": round(wpms * 1e3, 1),
                                  "tflops": round(wtf, 1),
                                  "roofline": {"bound": "mfma", "achieved": round(wtf, 1), "peak": BF16_PEAK_TFLOPS,
                                               "unit": "TFLOP/s", "frac": round(wtf / BF16_PEAK_TFLOPS, 4),
                                               "traffic": None,
                                               "kernel": "prefill_mfma_kernel<NW=4, paged> (paged_prefill_window)",
                                               "algorithmic_flops_per_launch": wflops},
                                  "flops_vs_no_window": round(wflops / cflops, 4)}
                log(f"windowed paged prefill {wpms * 1e3:.1f} us -> {wtf:.1f} TFLOP/s")
                window["paged_prefill"] = window_prefill
                del ckc, cvc, cq, cout
                torch.cuda.empty_cache()
    except Exception as e:  # a failing secondary figure must not cost the headline line
        log(f"window section failed: {e!r}")
        window = {"error": repr(e)}
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- FP8 cache
    fp8 = None
    try:
        if not args.no_fp8:
            t0 = time.perf_counter()
            fc = wl.make_case(8)
            fB, fHq, fHkv, fd = fc.spec.batch, fc.spec.num_q_heads, fc.spec.num_kv_heads, fc.spec.head_dim
            log(f"fp8 workload generated in {time.perf_counter() - t0:.1f}s: NB={fc.num_blocks}")
            fbytes = int(fc.context_lens.astype(np.int64).sum()) * fHkv * 2 * fd   # one byte per element
            fps = args.fp8_partition_size
            fP = ops.num_partitions(fc.max_context_len, fps)
            # the newest token of each sequence (its last row of the written history)
            last = np.cumsum(fc.context_lens.astype(np.int64)) - 1
            ks_d = torch.tensor([fc.k_scale], dtype=torch.float32, device=dev)
            vs_d = torch.tensor([fc.v_scale], dtype=torch.float32, device=dev)
            fk_all, fv_all, fslots = up(fc.k_new), up(fc.v_new), up(fc.slot_mapping)
            fcopies = []
            for _ in range(max(1, args.copies)):
                c = dict(q=up(fc.q), kc=up(fc.k_cache), vc=up(fc.v_cache), bt=up(fc.block_tables),
                         cl=up(fc.context_lens), kn=up(fc.k_new[last]), vn=up(fc.v_new[last]),
                         slots=up(fc.slot_mapping[last]),
                         po=torch.empty((fB, fHq, fP, fd), dtype=torch.float32, device=dev),
                         pl=torch.empty((fB, fHq, fP), dtype=torch.float32, device=dev),
                         out=torch.empty((fB, fHq, fd), dtype=torch.bfloat16, device=dev),
                         lse=torch.empty((fB, fHq), dtype=torch.float32, device=dev))
                ops.paged_kv_write(fk_all, fv_all, c["kc"], c["vc"], fslots, k_scale=ks_d, v_scale=vs_d)
                fcopies.append(c)
            # the quantising write of the whole history (bf16 rows in, E4M3 codes out),
            # rewritten into the first copy's pools (same values): HIP events around
            # 10 back-to-back writes after one warm-up
            ops.paged_kv_write(fk_all, fv_all, fcopies[0]["kc"], fcopies[0]["vc"], fslots, k_scale=ks_d, v_scale=vs_d)
            hwa, hwb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            hwa.record(stream)
            for _ in range(10):
                ops.paged_kv_write(fk_all, fv_all, fcopies[0]["kc"], fcopies[0]["vc"], fslots, k_scale=ks_d, v_scale=vs_d)
            hwb.record(stream)
            torch.cuda.synchronize()
            fw_ms = hwa.elapsed_time(hwb) / 10
            fw_tokens = int(fk_all.shape[0])
            fw_bytes = fw_tokens * fHkv * fd * 2 * 3   # K and V: 2 bytes read, 1 byte written per element
            del fk_all, fv_all

            def fdecode(c):
                ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], fc.max_context_len, fc.scale,
                                           fps, part_out=c["po"], part_lse=c["pl"], k_scale=ks_d, v_scale=vs_d)

            def fstep(c):
                ops.paged_attention_decode(c["q"], c["kc"], c["vc"], c["bt"], c["cl"], fc.max_context_len, fc.scale,
                                           fps, part_out=c["po"], part_lse=c["pl"], k_scale=ks_d, v_scale=vs_d,
                                           k_new=c["kn"], v_new=c["vn"])
                ops.paged_attention_reduce(c["po"], c["pl"], c["cl"], fps, out=c["out"], lse=c["lse"])

            def ftimed(fn, n_groups):
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(n_groups)]
                torch.cuda.synchronize()
                for gi in range(n_groups):
                    evs[gi][0].record(stream)
                    for k in range(group):
                        fn(fcopies[(gi * group + k) % len(fcopies)])
                    evs[gi][1].record(stream)
                torch.cuda.synchronize()
                return [a.elapsed_time(b) / group for a, b in evs]
            for i in range(args.warmup):
                fstep(fcopies[i % len(fcopies)])
            fg = max(1, args.steps // group)
            fdec_ms = ftimed(fdecode, fg)
            fstep_ms = ftimed(fstep, fg)
            favg = float(np.mean(fdec_ms))
            fgbs = fbytes / (favg * 1e-3) / 1e9
            fsms = float(np.mean(fstep_ms))
            fp8 = {"workload": fc.spec.name, "partition_size": fps, "k_scale": fc.k_scale, "v_scale": fc.v_scale,
                   "sum_context": int(fc.context_lens.sum()), "kv_bytes_per_step": fbytes,
                   "step_us": round(fsms * 1e3, 2), "step_gbs": round(fbytes / (fsms * 1e-3) / 1e9, 1),
                   "decode_tokens_per_s": round(fB / (fsms * 1e-3), 1),
                   "history_write": {"tokens": fw_tokens, "kernel_avg_us": round(fw_ms * 1e3, 1),
                                     "gbs": round(fw_bytes / (fw_ms * 1e-3) / 1e9, 1),
                                     "kernel": "kv_write_fp8_kernel<bf16> (paged_kv_write_fp8)",
                                     "bound": "vector arithmetic of the quantiser (16 correctly rounded divisions per 16-byte chunk of codes)"},
                   "roofline": {"bound": "hbm", "achieved": round(fgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(fgbs / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic(FP8_TRAFFIC_FILE, DECODE_SOURCES),
                                "kernel": "decode_mfma_kernel<G=4,BS=16,W=1,KV8> (paged_attention_decode_fp8)",
                                "kernel_avg_us": round(favg * 1e3, 2),
                                "timing": "HIP events on the launch stream around groups of 10 back-to-back launches",
                                "algorithmic_bytes_per_launch": fbytes}}
            log(f"fp8 decode kernel {favg * 1e3:.1f} us -> {fgbs:.0f} GB/s of E4M3 KV; step {fsms * 1e3:.1f} us; "
                f"history write ({fw_tokens} tokens) {fw_ms * 1e3:.1f} us -> {fw_bytes / (fw_ms * 1e-3) / 1e9:.0f} GB/s")
            if not args.no_cpu_baseline:
                try:
                    fp8["cpu_baseline"] = fp8_cpu_baseline(fc, min(args.cpu_seconds, 5.0))
                    log(f"fp8 decode cpu baseline {fp8['cpu_baseline']['value']} GB/s")
                except Exception as e:
                    log(f"fp8 cpu baseline failed: {e!r}")
            del fcopies
            torch.cuda.empty_cache()
    except Exception as e:  # a failing secondary figure must not cost the headline line
        log(f"fp8 section failed: {e!r}")
        fp8 = {"error": repr(e)}
        torch.cuda.empty_cache()

    # ---------------------------------------------- workloads 4 and 5 (decode)
    def decode_workload(cfg, n_copies, traffic_file, kernel_name):
        t0 = time.perf_counter()
        xc = wl.make_case(cfg)
        xs = xc.spec
        log(f"workload {cfg} generated in {time.perf_counter() - t0:.1f}s: NB={xc.num_blocks} "
            f"sum(ctx)={int(xc.context_lens.sum())}")
        xB, xHq, xHkv, xd, xbs, xps = (xs.batch, xs.num_q_heads, xs.num_kv_heads, xs.head_dim, xs.block_size,
                                       xs.partition_size)
        xmax = xc.max_context_len
        xP = ops.num_partitions(xmax, xps) if xps else 1
        ctx64 = xc.context_lens.astype(np.int64)
        logical = int(ctx64.sum()) * xHkv * 2 * xd * 2
        if xs.share_group:
            shared = xs.share_blocks * xbs
            unique = (xB // xs.share_group * shared + int((ctx64 - shared).sum())) * xHkv * 2 * xd * 2
        else:
            unique = logical
        bt, cl = up(xc.block_tables), up(xc.context_lens)
        xcopies = []
        for _ in range(n_copies):
            xcopies.append(dict(q=up(xc.q), kc=up(xc.k_cache), vc=up(xc.v_cache),
                                po=torch.empty((xB, xHq, xP, xd), dtype=torch.float32, device=dev),
                                pl=torch.empty((xB, xHq, xP), dtype=torch.float32, device=dev),
                                out=torch.empty((xB, xHq, xd), dtype=torch.bfloat16, device=dev),
                                lse=torch.empty((xB, xHq), dtype=torch.float32, device=dev)))

        def xdecode(i, ps=xps):
            c = xcopies[i]
            if ps:
                ops.paged_attention_decode(c["q"], c["kc"], c["vc"], bt, cl, xmax, xc.scale, ps,
                                           part_out=c["po"], part_lse=c["pl"])
            else:
                ops.paged_attention_decode(c["q"], c["kc"], c["vc"], bt, cl, xmax, xc.scale,
                                           out=c["out"], lse=c["lse"])

        def xstep(i):
            xdecode(i)
            if xps:
                c = xcopies[i]
                ops.paged_attention_reduce(c["po"], c["pl"], cl, xps, out=c["out"], lse=c["lse"])
        for i in range(4):
            xstep(i % n_copies)
        ng = max(2, args.steps // 40)
        dms = timed_groups(torch, stream, xdecode, n_copies, ng)
        sms = timed_groups(torch, stream, xstep, n_copies, ng)
        # a one-pass workload: the split kernel at 512-token partitions beside it
        split = {}
        if not xps:
            sP = ops.num_partitions(xmax, 512)
            for c in xcopies:
                c["po"] = torch.empty((xB, xHq, sP, xd), dtype=torch.float32, device=dev)
                c["pl"] = torch.empty((xB, xHq, sP), dtype=torch.float32, device=dev)
            xdecode(0, 512)
            vms = timed_groups(torch, stream, lambda i: xdecode(i, 512), n_copies, ng)
            split = {"512": {"kernel_avg_us": round(float(np.mean(vms)) * 1e3, 2),
                             "gbs_unique": round(unique / (float(np.mean(vms)) * 1e-3) / 1e9, 1)}}
        davg, savg = float(np.mean(dms)), float(np.mean(sms))
        ugbs = unique / (davg * 1e-3) / 1e9
        res = {"workload": xs.name, "batch": xB, "num_q_heads": xHq, "num_kv_heads": xHkv, "block_size": xbs,
               "partition_size": xps, "sum_context": int(ctx64.sum()), "num_blocks": xc.num_blocks,
               "input_copies": n_copies, "kv_bytes_unique": unique, "kv_bytes_logical": logical,
               "step_us": round(savg * 1e3, 2), "step_gbs_unique": round(unique / (savg * 1e-3) / 1e9, 1),
               "logical_gbs": round(logical / (davg * 1e-3) / 1e9, 1),
               "decode_tokens_per_s": round(xB / (savg * 1e-3), 1),
               "roofline": {"bound": "hbm", "achieved": round(ugbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(ugbs / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(traffic_file, DECODE_SOURCES),
                            "kernel": kernel_name, "kernel_avg_us": round(davg * 1e3, 2),
                            "kernel_median_us": round(float(np.median(dms)) * 1e3, 2),
                            "kernel_p10_us": round(float(np.percentile(dms, 10)) * 1e3, 2),
                            "kernel_p90_us": round(float(np.percentile(dms, 90)) * 1e3, 2),
                            "timing": "HIP events on the launch stream around groups of 10 back-to-back launches",
                            "algorithmic_bytes_per_launch": unique}}
        if split:
            res["roofline"]["partition_size_variants"] = split
        log(f"workload {cfg}: decode kernel {davg * 1e3:.1f} us -> {ugbs:.0f} GB/s unique "
            f"({logical / (davg * 1e-3) / 1e9:.0f} logical); step {savg * 1e3:.1f} us")
        del xcopies, bt, cl
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = decode_cpu_baseline(xc, min(args.cpu_seconds, 5.0))
            log(f"workload {cfg} cpu baseline {res['cpu_baseline']['value']} GB/s")
        return res

    # the pools of one copy (2.5-2.7 GB) exceed the Infinity Cache many times over
    def guarded_workload(cfg, *rest):
        try:
            return decode_workload(cfg, *rest)
        except Exception as e:  # a failing secondary figure must not cost the headline line
            log(f"workload {cfg} failed: {e!r}")
            torch.cuda.empty_cache()
            return {"error": repr(e)}
    c4 = None if args.no_c4 else guarded_workload(
        4, 2, C4_TRAFFIC_FILE, "decode_mfma_kernel<G=8,BS=32,W=4> (paged_attention_decode, one pass)")
    c5 = None if args.no_c5 else guarded_workload(
        5, 1, C5_TRAFFIC_FILE, "decode_mfma_kernel<G=4,BS=16,W=1> (paged_attention_decode) + reduce_kernel")

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n_blas = blas_threads()
        t0 = time.perf_counter()
        kc, vc = oracle.kv_write(case.k_cache, case.v_cache, case.k_new, case.v_new, case.slot_mapping, bs)
        n_done = 0
        bytes_done = 0
        while time.perf_counter() - t0 < args.cpu_seconds:  # whole sequences, ~10 s of CPU work
            b = n_done % B
            oracle.decode(case.q[b:b + 1], kc, vc, case.block_tables[b:b + 1], case.context_lens[b:b + 1],
                          bs, case.scale, spec.dtype)
            n_done += 1
            bytes_done += int(case.context_lens[b]) * Hkv * 2 * d * 2
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(bytes_done / cpu_s / 1e9, 4), "unit": "GB/s", "cores": int(n_blas),
               "kind": "oracle",
               "sample": f"fp64 NumPy oracle on the same workload: paged write of the 64 new tokens, "
                         f"then decode of {n_done} sequences in order, cycling over the 64 "
                         f"({n_done / B:.1f} passes, {bytes_done / 1e6:.1f} MB of KV) in {cpu_s:.2f} s; "
                         f"BLAS threads {n_blas}, {host_note()}"}
        log(f"cpu baseline {cpu['value']} GB/s on {n_done} sequences")

    line = {
        "metric": METRIC,
        "value": round(value_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "block_size": bs, "context_lens": "uniform[128,2048], seed 1002",
                   "sum_context": int(case.context_lens.sum()), "num_blocks": case.num_blocks,
                   "partition_size": ps, "input_copies": len(range(max(1, args.copies))),
                   "step": "paged_attention_decode_append (the 64 new tokens' cache write folded in) + "
                           "paged_attention_reduce",
                   "ms_per_step_three_launches": round(sep_ms, 5),
                   "graph_ms_per_step": g2 and round(g2, 5),
                   "graph_ms_per_step_three_launches": g3 and round(g3, 5),
                   "kv_bytes_per_step": kv_bytes},
        "roofline": roofline,
        "decode_tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "stream_ceiling": stream_ceiling,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "window": window,
        "fp8": fp8,
        "c4": c4,
        "c5": c5,
        "library_build_id": build_id,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
