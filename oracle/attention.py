"""fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or links
anything under ``oracle/``, and this module imports nothing from it.

What it computes is the plain definition of attention, written out with no
tiling, fusion or reordering: FlashAttention-style tiling and PagedAttention's
block indirection change where data sits and the order of the sums, not the
result ("Llama 4 inference doubling (FlashAttention-3 + PagedAttention +
vLLM)", section 3.1: the cache is one logical address space split into pages;
"LLaMA inference performance: structure and source", section 3.1: the six
steps of the attention forward).  So every function below is that definition
applied to the rows the paging model selects.

Inputs are the exact bytes the GPU receives: bf16 arrives as uint16 bit
patterns and is widened exactly; everything is computed in float64.

Readings of points the pages leave open:
  * query head h uses KV head h // G with G = H_q / H_kv (contiguous groups,
    which is what repeating each KV head G times yields; LLaMA page, 2.1/3.1);
  * the context length counts the token just written: the query sits at
    position ctx-1 and attends to positions 0..ctx-1;
  * lse is the natural log of the sum of exp(scores) over unmasked keys;
  * an empty key set gives out = 0 and lse = -inf;
  * a partition i covers positions [i*P, min((i+1)*P, ctx)); empty ones carry
    lse = -inf and weight 0 in the log-sum-exp merge;
  * prefill uses one cu_seqlens for q and k: row i of a sequence sees keys
    0..i of the same sequence;
  * paged prefill (a chunk of Lq new rows against ctx cached positions, the
    chunk's own K/V already written): the chunk is the last Lq positions,
    so row i sees positions 0..ctx-Lq+i (the causal mask aligned to the end);
  * a sliding window of W keys (0 = none) keeps positions max(0, p-W+1)..p
    for a query at position p; a split partition wholly before the window is
    empty (out 0, lse -inf), and the window-aware merge starts at the first
    partition the window reaches;
  * keys before the window take no part in any sum, so their blocks are
    never fetched: their table entries may name freed blocks (any value).

Every function here is pinned by tests/test_oracle_pins.py (closed forms,
torch SDPA, invariants, brute force), and tests/test_oracle_mutants.py plants
plausible slips in them and checks that a pin catches each: nothing is left
parity-unpinned.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3, e4m3_value

F32 = "f32"
BF16 = "bf16"


def upcast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening to float64 (bf16 given as uint16 bit patterns, E4M3
    as uint8 codes, widened to their unscaled values)."""
    if dtype == E4M3:
        return e4m3_value(x)
    if dtype == BF16:
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# a1: cache write
# ---------------------------------------------------------------------------
def kv_write(k_cache, v_cache, k, v, slot_mapping, block_size):
    """In-place style update of the paged pools, returned as new arrays.

    Token t with slot s >= 0 lands in physical block s // block_size at offset
    s % block_size, for every KV head; a negative slot is skipped.  This is
    the in-place update through the block table of "LLM inference
    optimisation: KV cache to FlashAttention", section 3.1 (step 2), with a
    slot standing for (physical block, offset).  The copy is of raw element
    bits: no arithmetic touches the values.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        kc[blk, :, off, :] = k[t]
        vc[blk, :, off, :] = v[t]
    return kc, vc


# ---------------------------------------------------------------------------
# a0 / a2: logical -> physical gather through the block table
# ---------------------------------------------------------------------------
def gather(pool, table_row, ctx, block_size, start=0):
    """Rows start..ctx-1 of one sequence, fetched through its block table.

    Logical page p // block_size maps to the physical block the table names
    ("Llama 4 inference doubling ...", section 3.1: logical page number to
    physical block number, int32, -1 = unallocated).  Returns
    ``[ctx - start, H_kv, d]`` in the pool's storage dtype; pages before
    ``start`` are not looked up.
    """
    num_blocks = pool.shape[0]
    rows = []
    for p in range(int(start), int(ctx)):
        blk = int(table_row[p // block_size])
        if not 0 <= blk < num_blocks:
            raise IndexError(f"position {p}: block id {blk} outside [0, {num_blocks})")
        rows.append(pool[blk, :, p % block_size, :])
    if not rows:
        return np.zeros((0, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    return np.stack(rows)


# ---------------------------------------------------------------------------
# a3 + a4: the plain attention of one query row
# ---------------------------------------------------------------------------
def attend(q, K, V, scale):
    """softmax(scale * K q) weighted sum of V, for one query row.

    Follows the LLaMA page's section 3.1: scores are q.k times the scale
    (step 3), masked keys are simply absent from K (step 4), softmax over the
    keys (step 5, here in float64), weighted sum of V (step 6).  Returns
    (out [d], lse, probabilities [n]); lse = log(sum(exp(scores))) in natural
    log.  The max is subtracted before exp only to keep exp finite; it
    cancels exactly in the quotient.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -math.inf, np.zeros(0)
    scores = scale * (K @ q)
    m = scores.max()
    w = np.exp(scores - m)
    z = w.sum()
    probs = w / z
    out = probs @ V
    lse = m + math.log(z)
    return out, lse, probs


def group_of(h, num_q_heads, num_kv_heads):
    """KV head serving query head h: contiguous groups of G = H_q / H_kv."""
    G = num_q_heads // num_kv_heads
    return h // G


# ---------------------------------------------------------------------------
# decode: each sequence's query against its paged history
# ---------------------------------------------------------------------------
def kv_rows(rows, dtype, kv_dtype, scale):
    """Gathered cache rows as float64: widened in the input dtype, or for an
    E4M3 cache the code values times the pool's fp32 scale."""
    if kv_dtype is None:
        return upcast(rows, dtype)
    return upcast(rows, kv_dtype) * float(np.float32(scale))


def window_start(pos, window):
    """First key a query at position pos sees under a sliding window of
    `window` keys (0 = no window): max(0, pos - window + 1), the row mask of
    "PageAttention + FlashAttention golden combination", section 4.1."""
    return max(0, int(pos) - int(window) + 1) if window > 0 else 0


def decode(q, k_cache, v_cache, block_tables, context_lens, block_size, scale,
           dtype, return_probs=False, window=0, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """PagedAttention decode for a batch: out [B, H_q, d] float64, lse [B, H_q].

    Each new token attends over its sequence's whole history, gathered block
    by block through the table ("PageAttention + FlashAttention golden
    combination", section 2.1; LLaMA page, section 3.2), with query heads
    sharing KV heads in groups (LLaMA page, section 2.1).  With a sliding
    window only the last `window` positions are seen.  ``kv_dtype`` = E4M3:
    the pools hold E4M3 codes, read as code value times k_scale / v_scale.
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -math.inf)
    probs = {}
    for b in range(B):
        ctx = int(context_lens[b])
        lo = window_start(ctx - 1, window) if ctx > 0 else 0
        Kall = kv_rows(gather(k_cache, block_tables[b], ctx, block_size, lo), dtype, kv_dtype, k_scale)
        Vall = kv_rows(gather(v_cache, block_tables[b], ctx, block_size, lo), dtype, kv_dtype, v_scale)
        for h in range(Hq):
            g = group_of(h, Hq, Hkv)
            o, l, p = attend(upcast(q[b, h], dtype), Kall[:, g, :], Vall[:, g, :], scale)
            out[b, h], lse[b, h] = o, l
            probs[(b, h)] = p
    if return_probs:
        return out, lse, probs
    return out, lse


# ---------------------------------------------------------------------------
# split-KV partitions and their log-sum-exp merge
# ---------------------------------------------------------------------------
def num_partitions(max_context_len, partition_size):
    return max(1, -(-int(max_context_len) // int(partition_size)))


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens,
                      block_size, scale, dtype, partition_size,
                      max_partitions=None, window=0, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Attention restricted to each partition of positions.

    Returns part_out [B, H_q, P, d] and part_lse [B, H_q, P]; a partition that
    holds no visible position of the sequence (past its end, or wholly before
    a sliding window) has out 0 and lse -inf.
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    P = max_partitions or num_partitions(int(context_lens.max()), partition_size)
    part_out = np.zeros((B, Hq, P, d))
    part_lse = np.full((B, Hq, P), -math.inf)
    for b in range(B):
        ctx = int(context_lens[b])
        wlo = window_start(ctx - 1, window) if ctx > 0 else 0
        # Kall[i] holds position wlo + i
        Kall = kv_rows(gather(k_cache, block_tables[b], ctx, block_size, wlo), dtype, kv_dtype, k_scale)
        Vall = kv_rows(gather(v_cache, block_tables[b], ctx, block_size, wlo), dtype, kv_dtype, v_scale)
        for i in range(P):
            lo, hi = max(i * partition_size, wlo), min((i + 1) * partition_size, ctx)
            if lo >= hi:
                continue
            for h in range(Hq):
                g = group_of(h, Hq, Hkv)
                o, l, _ = attend(upcast(q[b, h], dtype), Kall[lo - wlo:hi - wlo, g, :],
                                 Vall[lo - wlo:hi - wlo, g, :], scale)
                part_out[b, h, i], part_lse[b, h, i] = o, l
    return part_out, part_lse


def reduce_partitions(part_out, part_lse, context_lens, partition_size, window=0):
    """Merge partition results by log-sum-exp.

    With M the largest partition lse and w_i = exp(lse_i - M) (0 for a
    partition past the end of the sequence), the merged output is
    sum_i w_i o_i / sum_i w_i and the merged lse is M + log(sum_i w_i).  The
    LSE that the varlen interface returns ("Llama 4 inference doubling ...",
    section 2.4) is what makes this merge exact.  With a sliding window the
    merge starts at the partition holding the window's first key: the ones
    before it are empty by definition and are not read.
    """
    B, Hq, P, d = part_out.shape
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        ctx = int(context_lens[b])
        live = min(P, -(-ctx // int(partition_size)))
        first = window_start(ctx - 1, window) // int(partition_size) if ctx > 0 else 0
        if live <= first:
            continue
        for h in range(Hq):
            l = np.asarray(part_lse[b, h, first:live], dtype=np.float64)
            M = l.max()
            if M == -math.inf:
                continue
            w = np.exp(l - M)
            W = w.sum()
            out[b, h] = (w[:, None] * np.asarray(part_out[b, h, first:live], dtype=np.float64)).sum(0) / W
            lse[b, h] = M + math.log(W)
    return out, lse


# ---------------------------------------------------------------------------
# varlen causal prefill
# ---------------------------------------------------------------------------
def prefill(q, k, v, cu_seqlens, scale, dtype, heads=None, seqs=None, window=0):
    """Causal self-attention of each packed sequence: out [T, H_q, d], lse [T, H_q].

    Sequences are packed back to back and delimited by the cumulative length
    array, with no padding ("Llama 4 inference doubling ...", section 2.4,
    the varlen call with causal=True returning out and lse).  Within sequence
    s, row i sees keys 0..i of the same sequence: the causal mask of the
    LLaMA page's section 3.1 step 4, built with -inf so masked keys get
    weight 0.  With a sliding window row i also loses keys before
    i - window + 1 ("PageAttention + FlashAttention golden combination",
    section 4.1).  ``heads``/``seqs`` restrict the computation to a subset.
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -math.inf)
    S = len(cu_seqlens) - 1
    for s in (range(S) if seqs is None else seqs):
        a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        L = e - a
        if L <= 0:
            continue
        for h in (range(Hq) if heads is None else heads):
            g = group_of(h, Hq, Hkv)
            Q = upcast(q[a:e, h, :], dtype)
            K = upcast(k[a:e, g, :], dtype)
            V = upcast(v[a:e, g, :], dtype)
            scores = scale * (Q @ K.T)                       # [L, L]
            future = np.triu(np.ones((L, L), dtype=bool), 1)  # key j > row i
            scores[future] = -np.inf
            if window > 0:
                scores[np.tril(np.ones((L, L), dtype=bool), -window)] = -np.inf  # key j <= i - window
            m = scores.max(axis=1, keepdims=True)
            w = np.exp(scores - m)
            z = w.sum(axis=1, keepdims=True)
            out[a:e, h, :] = (w / z) @ V
            lse[a:e, h] = (m + np.log(z))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# paged prefill: a new chunk of queries against a cached prefix plus itself
# ---------------------------------------------------------------------------
def paged_prefill(q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens,
                  block_size, scale, dtype, heads=None, seqs=None, window=0):
    """Chunked / prefix-cached prefill: out [T_q, H_q, d], lse [T_q, H_q].

    The varlen call takes separate cumulative lengths for queries and keys
    with causal=True ("Llama 4 inference doubling ...", section 2.4), and the
    engine reuses cached KV of earlier requests (prefix caching, same page,
    section 4.2).  Here the keys of sequence s are its first context_lens[s]
    cache positions, fetched through its block table (section 3.1 paging),
    and its Lq = cu_seqlens_q[s+1] - cu_seqlens_q[s] query rows are the last
    Lq of those positions (their own K/V already written): row i sits at
    position ctx - Lq + i and sees keys 0 .. ctx - Lq + i (with a sliding
    window, only the last `window` of those).
    """
    T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -math.inf)
    S = len(cu_seqlens_q) - 1
    for s in (range(S) if seqs is None else seqs):
        a, e = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        Lq = e - a
        ctx = int(context_lens[s])
        if Lq <= 0:
            continue
        if Lq > ctx:
            raise ValueError(f"sequence {s}: {Lq} query rows but only {ctx} cached positions")
        # the first row's window start: no row sees a key before it
        k0 = window_start(ctx - Lq, window)
        keys = np.arange(k0, ctx)[None, :]                               # key positions
        for h in (range(Hq) if heads is None else heads):
            g = group_of(h, Hq, Hkv)
            K = upcast(gather(k_cache[:, g:g + 1], block_tables[s], ctx, block_size, k0), dtype)[:, 0, :]
            V = upcast(gather(v_cache[:, g:g + 1], block_tables[s], ctx, block_size, k0), dtype)[:, 0, :]
            Q = upcast(q[a:e, h, :], dtype)
            scores = scale * (Q @ K.T)                                   # [Lq, ctx - k0]
            pos = ctx - Lq + np.arange(Lq)[:, None]                      # row positions
            scores[keys > pos] = -np.inf
            if window > 0:
                scores[keys <= pos - window] = -np.inf
            m = scores.max(axis=1, keepdims=True)
            w = np.exp(scores - m)
            z = w.sum(axis=1, keepdims=True)
            out[a:e, h, :] = (w / z) @ V
            lse[a:e, h] = (m + np.log(z))[:, 0]
    return out, lse
