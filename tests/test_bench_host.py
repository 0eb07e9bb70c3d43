"""The benchmark's host side, on the CPU: the one-GPU refusal, the oracle
baselines it times beside each GPU figure (their fields and their byte
accounting, on small cases), and the committed counter traffic it reports
(present for the sources as they stand, withheld once they change).
"""
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import bench
from attention_paged_kv_write_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _fields(r, unit):
    assert r["unit"] == unit and r["kind"] == "oracle"
    assert r["value"] > 0 and r["cores"] >= 1 and r["sample"]


def _decoded(r):
    """(sequences decoded, MB of KV counted) from a decode baseline's sample."""
    m = re.search(r"decode of (\d+) sequences in order \(([\d.]+) MB of KV\)", r["sample"])
    assert m, r["sample"]
    return int(m.group(1)), float(m.group(2))


def _want_mb(ctx, n, nseq, per_pos, window=0):
    vis = np.minimum(ctx, window) if window else ctx
    return sum(int(vis[i % nseq]) for i in range(n)) * per_pos / 1e6


def test_decode_baseline_counts_the_kv_of_each_sequence_decoded():
    case = wl.make_case(2, batch=4, ctx_min=20, ctx_max=200, max_blocks_per_seq=13)
    r = bench.decode_cpu_baseline(case, 0.3)
    _fields(r, "GB/s")
    n, mb = _decoded(r)
    per_pos = case.spec.num_kv_heads * 2 * case.spec.head_dim * 2
    assert n >= 1 and abs(mb - _want_mb(case.context_lens.astype(np.int64), n, 4, per_pos)) <= 0.051


def test_window_baseline_counts_only_the_window():
    case = wl.make_case(7, batch=4, ctx_min=20, ctx_max=300, max_blocks_per_seq=19, window=64)
    assert (case.context_lens > 64).any()
    r = bench.window_cpu_baseline(case, 64, 0.3)
    _fields(r, "GB/s")
    n, mb = _decoded(r)
    per_pos = case.spec.num_kv_heads * 2 * case.spec.head_dim * 2
    assert abs(mb - _want_mb(case.context_lens.astype(np.int64), n, 4, per_pos, window=64)) <= 0.051


def test_fp8_baseline_counts_one_byte_per_element():
    case = wl.make_case(8, batch=4, ctx_min=10, ctx_max=100, max_blocks_per_seq=7)
    r = bench.fp8_cpu_baseline(case, 0.3, nseq=2)
    _fields(r, "GB/s")
    n, mb = _decoded(r)
    per_pos = case.spec.num_kv_heads * 2 * case.spec.head_dim
    assert abs(mb - _want_mb(case.context_lens.astype(np.int64), n, 2, per_pos)) <= 0.051
    assert "first 2 sequences" in r["sample"]


def test_prefill_baselines_report_tflops():
    pc = wl.make_case(3, num_seqs=3, lens_fixed=(5, 40, 17))
    r = bench.prefill_cpu_baseline(pc, 30.0)
    _fields(r, "TFLOP/s")
    assert "first 3 of 3 sequences (62 rows" in r["sample"]
    cc = wl.make_case(6, num_seqs=3, prefix_fixed=(0, 40, 100), chunk_fixed=(5, 30, 17))
    r = bench.paged_prefill_cpu_baseline(cc, 30.0)
    _fields(r, "TFLOP/s")
    assert "first 3 of 3 sequences (52 query rows" in r["sample"]


def test_rope_baseline_reports_gbs():
    pc = wl.make_case(3, num_seqs=3, lens_fixed=(5, 40, 17))
    cu = pc.cu_seqlens.astype(np.int64)
    pos = np.concatenate([np.arange(cu[i + 1] - cu[i]) for i in range(3)]).astype(np.int32)
    r = bench.rope_cpu_baseline(pc, pos, pc.spec.head_dim, 10000.0, 1000.0)
    _fields(r, "GB/s")
    assert "all 62 prompt rows" in r["sample"]


TRAFFIC = [
    (bench.DECODE_TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.C4_TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.C5_TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.FP8_TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.WINDOW_TRAFFIC_FILE, bench.DECODE_SOURCES),
    (bench.PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES),
    (bench.PAGED_PREFILL_TRAFFIC_FILE, bench.PREFILL_SOURCES),
    (bench.ROPE_TRAFFIC_FILE, bench.ROPE_SOURCES),
    (bench.KV_WRITE_TRAFFIC_FILE, bench.KV_WRITE_SOURCES),
]


@pytest.mark.parametrize("path,sources", TRAFFIC, ids=[os.path.basename(p) for p, _ in TRAFFIC])
def test_committed_traffic_matches_the_sources(path, sources):
    """Each committed traffic summary was taken on the kernel sources as they
    stand (else the bench reports no traffic for that kernel)."""
    t = bench.measured_traffic(path, sources)
    assert t is not None and t > 0, f"{os.path.basename(path)}: counters taken on other sources"


def test_traffic_is_withheld_for_other_sources(tmp_path):
    with open(bench.DECODE_TRAFFIC_FILE) as f:
        t = json.load(f)
    t["kernel_source_sha256"] = "0" * 64
    p = tmp_path / "stale.txt"
    p.write_text(json.dumps(t))
    assert bench.measured_traffic(str(p), bench.DECODE_SOURCES) is None
    assert bench.measured_traffic(str(tmp_path / "missing.txt"), bench.DECODE_SOURCES) is None
