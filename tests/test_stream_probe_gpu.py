"""GPU check of the paged stream probe (paged_kv_stream_read), the measurement
call that reads what a split decode reads and does no attention: its XOR
checksum of every K/V word per (sequence, KV head, partition) must equal the
same XOR taken on the host pools, bit for bit, in both fetch modes and at
every supported depth.  (Not attention: nothing here needs the oracle.)"""
import numpy as np
import pytest
import torch

from attention_paged_kv_write_amd import ops
from attention_paged_kv_write_amd import workloads as wl
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def host_checksums(case, partition_size):
    bs = case.spec.block_size
    B, Hkv = case.spec.batch, case.spec.num_kv_heads
    P = ops.num_partitions(case.max_context_len, partition_size)
    sums = {}
    for b in range(B):
        ctx = int(case.context_lens[b])
        for i in range(P):
            lo, hi = i * partition_size, min((i + 1) * partition_size, ctx)
            if lo >= hi:
                continue
            for g in range(Hkv):
                acc = np.uint32(0)
                for p in range(lo, hi):
                    blk = case.block_tables[b, p // bs]
                    for pool in (case.k_cache, case.v_cache):
                        acc ^= np.bitwise_xor.reduce(np.ascontiguousarray(pool[blk, g, p % bs]).view(np.uint32))
                sums[(b, g, i)] = int(acc)
    return sums


@pytest.mark.parametrize("cfg,over,ps", [
    (2, dict(batch=6, ctx_min=1, ctx_max=700, max_blocks_per_seq=44), 256),
    (4, dict(batch=8, ctx_min=520, ctx_max=1500, max_blocks_per_seq=47), 512),
    (2, dict(batch=3, block_size=64, ctx_min=1, ctx_max=500, max_blocks_per_seq=8), 128),
    (2, dict(batch=2, ctx_fixed=(2048 + 37, 1500), max_blocks_per_seq=131), 2048),   # 128 blocks per unit
])
def test_stream_checksums_match_pools(cfg, over, ps):
    case = wl.make_case(cfg, **over)
    want = host_checksums(case, ps)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    bt, cl = to_dev(case.block_tables), to_dev(case.context_lens)
    for mode, depths in ((ops.PA_STREAM_LDS_DMA, (2, 3, 4)), (ops.PA_STREAM_REGISTERS, (1, 2, 4))):
        for depth in depths:
            got = ops.paged_kv_stream_read(kc, vc, bt, cl, case.max_context_len, ps, mode, depth)
            torch.cuda.synchronize()
            g = got.cpu().numpy().view(np.uint32)
            for (b, h, i), v in want.items():
                assert int(g[b, h, i]) == v, (mode, depth, b, h, i)


def test_stream_rejects_unsupported():
    case = wl.make_case(2, batch=2, ctx_min=1, ctx_max=100, max_blocks_per_seq=7)
    kc, vc = to_dev(case.k_cache), to_dev(case.v_cache)
    bt, cl = to_dev(case.block_tables), to_dev(case.context_lens)
    with pytest.raises(ops.PagedAttnError):
        ops.paged_kv_stream_read(kc, vc, bt, cl, case.max_context_len, 64, ops.PA_STREAM_LDS_DMA, 5)
    with pytest.raises(ops.PagedAttnError):
        ops.paged_kv_stream_read(kc, vc, bt, cl, case.max_context_len, 24, ops.PA_STREAM_LDS_DMA, 2)


def host_contiguous_sums(words, waves):
    # wave w takes the 16-byte chunks [w*cpw, min((w+1)*cpw, n)), cpw = ceil(n / waves)
    n = words.size // 4
    cpw = -(-n // waves)
    out = np.zeros(waves, dtype=np.uint32)
    for w in range(waves):
        lo, hi = w * cpw, min((w + 1) * cpw, n)
        if lo < hi:
            out[w] = np.bitwise_xor.reduce(words[4 * lo:4 * hi])
    return out


@pytest.mark.parametrize("nbytes,waves", [(16, 1), (16 * 1000, 7), (16 * 64 * 9 + 16 * 5, 3),
                                          ((1 << 20) + 16 * 3, 64), (16 * 10, 32)])
def test_contiguous_read_checksums(nbytes, waves):
    rng = np.random.default_rng(nbytes + waves)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    want = host_contiguous_sums(words, waves)
    for depth in (1, 2, 4, 8):
        got = ops.stream_read_contiguous(src, waves=waves, depth=depth)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want, err_msg=f"depth {depth}")
