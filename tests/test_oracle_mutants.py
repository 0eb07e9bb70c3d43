"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant swaps one oracle function for a copy with one plausible slip (a
wrong group map, a dropped scale, a log in the wrong base, a transposed
index, an off-by-one in the mask or the context), then runs the pins of
test_oracle_pins.py against it and expects at least one to fail.  The real
oracle is restored after each case.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import test_oracle_pins as pins


def _attend_no_scale(q, K, V, scale):
    return oa.__dict__["_orig_attend"](q, K, V, 1.0)


def _attend_log2(q, K, V, scale):
    out, lse, p = oa.__dict__["_orig_attend"](q, K, V, scale)
    return out, lse / math.log(2.0), p


def _attend_drop_last_key(q, K, V, scale):
    if K.shape[0] > 1:
        K, V = K[:-1], V[:-1]
    return oa.__dict__["_orig_attend"](q, K, V, scale)


def _group_mod(h, num_q_heads, num_kv_heads):
    return h % (num_q_heads // num_kv_heads)


def _gather_swapped(pool, table_row, ctx, block_size, start=0):
    rows = []
    for p in range(int(start), int(ctx)):
        blk = int(table_row[p % block_size]) if p % block_size < len(table_row) else 0
        rows.append(pool[blk, :, p // block_size % block_size, :])
    if not rows:
        return np.zeros((0, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    return np.stack(rows)


def _kv_write_off_by_one(k_cache, v_cache, k, v, slot_mapping, block_size):
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    for t, s in enumerate(slot_mapping):
        if s < 0:
            continue
        blk, off = divmod(int(s), block_size)
        off = (off + 1) % block_size
        kc[blk, :, off, :] = k[t]
        vc[blk, :, off, :] = v[t]
    return kc, vc


def _prefill_mask(shift):
    def prefill(q, k, v, cu_seqlens, scale, dtype, heads=None, seqs=None):
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        out = np.zeros((T, Hq, d))
        lse = np.full((T, Hq), -math.inf)
        for s in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            L = e - a
            if L <= 0:
                continue
            for h in range(Hq):
                g = h // (Hq // Hkv)
                Q, K, V = (oa.upcast(q[a:e, h], dtype), oa.upcast(k[a:e, g], dtype),
                           oa.upcast(v[a:e, g], dtype))
                sc = scale * (Q @ K.T)
                sc[np.triu(np.ones((L, L), bool), shift)] = -np.inf
                m = sc.max(1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                w = np.exp(sc - m)
                z = w.sum(1, keepdims=True)
                out[a:e, h] = (w / z) @ V
                lse[a:e, h] = (m + np.log(z))[:, 0]
        return out, lse
    return prefill


def _paged_prefill_top_left(q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens,
                            block_size, scale, dtype, heads=None, seqs=None):
    # mask aligned to the first cached position instead of the chunk's own
    T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -math.inf)
    for s in range(len(cu_seqlens_q) - 1):
        a, e = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        ctx = int(context_lens[s])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            K = oa.upcast(oa.gather(k_cache[:, g:g + 1], block_tables[s], ctx, block_size), dtype)[:, 0]
            V = oa.upcast(oa.gather(v_cache[:, g:g + 1], block_tables[s], ctx, block_size), dtype)[:, 0]
            for i in range(e - a):
                o, l, _ = oa.attend(oa.upcast(q[a + i, h], dtype), K[:i + 1], V[:i + 1], scale)
                out[a + i, h], lse[a + i, h] = o, l
    return out, lse


def _window_start_off_by_one(pos, window):
    return max(0, int(pos) - int(window)) if window > 0 else 0


def _reduce_counts_dead(part_out, part_lse, context_lens, partition_size, window=0):
    B, Hq, P, d = part_out.shape
    return oa.__dict__["_orig_reduce"](part_out, part_lse, np.full(B, P * partition_size), partition_size,
                                       window)


def _reduce_window_skips_first_partition(part_out, part_lse, context_lens, partition_size, window=0):
    # the merge starts one partition late under a window
    lens = np.asarray(context_lens, dtype=np.int64)
    if window > 0:
        lens = np.where(lens > 0, lens, 0)
        shifted = np.maximum(lens - 1 - window + 1, 0) // partition_size
        po, pl = part_out.copy(), part_lse.copy()
        for b, f in enumerate(shifted):
            pl[b, :, :f + 1] = -np.inf
        return oa.__dict__["_orig_reduce"](po, pl, context_lens, partition_size, 0)
    return oa.__dict__["_orig_reduce"](part_out, part_lse, context_lens, partition_size, window)


def _upcast_bf16_as_integers(x, dtype):
    # bf16 bit patterns widened as if they were integer values
    if dtype == oa.BF16:
        return np.asarray(x).astype(np.float64)
    return oa.__dict__["_orig_upcast"](x, dtype)


def _decode_drops_newest(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, dtype,
                         return_probs=False, window=0, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    # the query attends to positions 0..ctx-2 (the token just written is left out)
    lens = np.maximum(np.asarray(context_lens) - 1, 1)
    return oa.__dict__["_orig_decode"](q, k_cache, v_cache, block_tables, lens, block_size, scale, dtype,
                                       return_probs, window, kv_dtype, k_scale, v_scale)


def _partitions_start_one_late(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, dtype,
                               partition_size, max_partitions=None, window=0, kv_dtype=None,
                               k_scale=1.0, v_scale=1.0):
    # every partition but the first starts one position late (its first key is lost)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    P = max_partitions or oa.num_partitions(int(np.max(context_lens)), partition_size)
    po = np.zeros((B, Hq, P, d))
    pl = np.full((B, Hq, P), -math.inf)
    for b in range(B):
        ctx = int(context_lens[b])
        K = oa.upcast(oa.gather(k_cache, block_tables[b], ctx, block_size), dtype)
        V = oa.upcast(oa.gather(v_cache, block_tables[b], ctx, block_size), dtype)
        for i in range(P):
            lo, hi = i * partition_size + (1 if i else 0), min((i + 1) * partition_size, ctx)
            if lo >= hi:
                continue
            for h in range(Hq):
                g = oa.group_of(h, Hq, Hkv)
                o, l, _ = oa.attend(oa.upcast(q[b, h], dtype), K[lo:hi, g], V[lo:hi, g], scale)
                po[b, h, i], pl[b, h, i] = o, l
    return po, pl


MUTANTS = {
    "bf16_widened_as_integers": [("upcast", _upcast_bf16_as_integers)],
    "decode_drops_newest_position": [("decode", _decode_drops_newest)],
    "partitions_start_one_late": [("decode_partitions", _partitions_start_one_late)],
    "group_map_h_mod_G": [("group_of", _group_mod)],
    "dropped_scale": [("attend", _attend_no_scale)],
    "lse_in_log2": [("attend", _attend_log2)],
    "context_off_by_one": [("attend", _attend_drop_last_key)],
    "gather_block_offset_swapped": [("gather", _gather_swapped)],
    "write_offset_off_by_one": [("kv_write", _kv_write_off_by_one)],
    "causal_mask_hides_diagonal": [("prefill", _prefill_mask(0))],
    "causal_mask_leaks_next_key": [("prefill", _prefill_mask(2))],
    "merge_counts_dead_partitions": [("reduce_partitions", _reduce_counts_dead)],
    "paged_prefill_mask_top_left": [("paged_prefill", _paged_prefill_top_left)],
    "window_one_key_too_many": [("window_start", _window_start_off_by_one)],
    "window_merge_skips_first_partition": [("reduce_partitions", _reduce_window_skips_first_partition)],
}

PIN_CALLS = [
    lambda g: pins.test_golden_kv_write(g),
    lambda g: pins.test_golden_attention_closed_form(g),
    lambda g: pins.test_golden_causal_prefill(g),
    lambda g: pins.test_golden_gqa_group_map(g),
    lambda g: pins.test_golden_lse_merge(g),
    lambda g: pins.test_decode_equals_unpaged_sdpa(4, 2, 64, 16, (1, 17, 33, 64)),
    lambda g: pins.test_needle_picks_one_value(63),
    lambda g: pins.test_single_key_returns_its_value(),
    lambda g: pins.test_prefill_equals_dense_causal_sdpa(),
    lambda g: pins.test_split_then_merge_equals_unsplit(48),
    lambda g: pins.test_paged_prefill_equals_masked_sdpa((7, 40, 100), (7, 13, 1), 16),
    lambda g: pins.test_window_decode_equals_masked_sdpa_and_split_merge(7),
    lambda g: pins.test_window_decode_equals_masked_sdpa_and_split_merge(40),
    lambda g: pins.test_decode_bf16_upcast_exact(),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, golden_dir, monkeypatch):
    monkeypatch.setitem(oa.__dict__, "_orig_attend", oa.attend)
    monkeypatch.setitem(oa.__dict__, "_orig_reduce", oa.reduce_partitions)
    monkeypatch.setitem(oa.__dict__, "_orig_upcast", oa.upcast)
    monkeypatch.setitem(oa.__dict__, "_orig_decode", oa.decode)
    for fn_name, repl in MUTANTS[name]:
        monkeypatch.setattr(oa, fn_name, repl)
        if hasattr(oracle, fn_name):
            monkeypatch.setattr(oracle, fn_name, repl)
    caught = 0
    for call in PIN_CALLS:
        try:
            with np.errstate(all="ignore"):
                call(golden_dir)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_every_pin(golden_dir):
    for call in PIN_CALLS:
        call(golden_dir)
