"""Pure-Python scalar loops for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``).  This is a
second, independent spelling of the same definitions, using Python floats,
``math.exp`` and ``math.log`` only, with no NumPy arithmetic, so that a slip
in the vectorised oracle (an index, a transposed operand, a dropped term) has
something other than itself to disagree with.  Inputs are plain nested lists
of Python floats (the caller widens bf16/fp32 exactly beforehand).
"""
from __future__ import annotations

import math


def softmax_attend(q, keys, values, scale):
    """One query row against lists of key/value rows: (out, lse)."""
    n = len(keys)
    if n == 0:
        return [0.0] * len(values[0]) if values else [], -math.inf
    scores = []
    for j in range(n):
        acc = 0.0
        for e in range(len(q)):
            acc += q[e] * keys[j][e]
        scores.append(acc * scale)
    big = max(scores)
    weights = [math.exp(s - big) for s in scores]
    total = 0.0
    for w in weights:
        total += w
    d = len(values[0])
    out = [0.0] * d
    for j in range(n):
        for e in range(d):
            out[e] += weights[j] * values[j][e]
    out = [x / total for x in out]
    return out, big + math.log(total)


def paged_decode(q, k_pool, v_pool, tables, ctx_lens, block_size, scale):
    """q [B][Hq][d]; pools [NB][Hkv][bs][d]; tables [B][M]; returns out, lse."""
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k_pool[0])
    group = Hq // Hkv
    out, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            g = h // group
            keys, values = [], []
            for p in range(ctx_lens[b]):
                blk = tables[b][p // block_size]
                keys.append(k_pool[blk][g][p % block_size])
                values.append(v_pool[blk][g][p % block_size])
            o, l = softmax_attend(q[b][h], keys, values, scale)
            ob.append(o)
            lb.append(l)
        out.append(ob)
        lse.append(lb)
    return out, lse


def causal_prefill(q, k, v, cu_seqlens, scale):
    """q [T][Hq][d], k/v [T][Hkv][d]; returns out [T][Hq][d], lse [T][Hq]."""
    T = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    group = Hq // Hkv
    out = [[None] * Hq for _ in range(T)]
    lse = [[None] * Hq for _ in range(T)]
    for s in range(len(cu_seqlens) - 1):
        start, end = cu_seqlens[s], cu_seqlens[s + 1]
        for i in range(start, end):
            for h in range(Hq):
                g = h // group
                keys = [k[j][g] for j in range(start, i + 1)]
                values = [v[j][g] for j in range(start, i + 1)]
                out[i][h], lse[i][h] = softmax_attend(q[i][h], keys, values, scale)
    return out, lse


def write_slots(k_pool, v_pool, k_new, v_new, slots, block_size):
    """Copy rows into the pools by slot; returns new nested lists."""
    kp = [[[list(r) for r in hh] for hh in blk] for blk in k_pool]
    vp = [[[list(r) for r in hh] for hh in blk] for blk in v_pool]
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk = s // block_size
        off = s - blk * block_size
        for h in range(len(k_new[t])):
            kp[blk][h][off] = list(k_new[t][h])
            vp[blk][h][off] = list(v_new[t][h])
    return kp, vp


def paged_prefill(q, k_pool, v_pool, tables, cu_q, ctx_lens, block_size, scale):
    """q [T][Hq][d]; pools [NB][Hkv][bs][d]; row i of sequence s (Lq rows, ctx
    keys) sees positions 0 .. ctx - Lq + i; returns out [T][Hq][d], lse [T][Hq]."""
    T = len(q)
    Hq = len(q[0])
    Hkv = len(k_pool[0])
    group = Hq // Hkv
    out = [[None] * Hq for _ in range(T)]
    lse = [[None] * Hq for _ in range(T)]
    for s in range(len(cu_q) - 1):
        start, end = cu_q[s], cu_q[s + 1]
        lq = end - start
        for i in range(lq):
            last = ctx_lens[s] - lq + i
            for h in range(Hq):
                g = h // group
                keys, values = [], []
                for p in range(last + 1):
                    blk = tables[s][p // block_size]
                    keys.append(k_pool[blk][g][p % block_size])
                    values.append(v_pool[blk][g][p % block_size])
                out[start + i][h], lse[start + i][h] = softmax_attend(q[start + i][h], keys, values, scale)
    return out, lse
