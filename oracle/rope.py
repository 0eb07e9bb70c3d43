"""fp64 CPU oracle for rotary position embedding fused into the cache write.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it.  It shares no code with the HIP path.

"LLaMA inference performance: structure and source" (section 2.2) describes
RoPE as a rotation, in complex space, of every query and key vector by an
amount set by its position, computed with sin and cos and worth caching as a
precomputed table; its attention listing applies it first (step 1 of section
3.1, `apply_rotary_pos_emb(query, key, cos, sin, position_ids)` with cos and
sin from the model's rotary-embedding table).  The pages print neither the
frequencies nor how dims are paired.  Readings taken here:
  * the rotated dims are the first `rot_dim` of each head (rot_dim even,
    rot_dim <= head_dim; LLaMA rotates all of them); the rest pass through;
  * dims i and i + rot_dim/2 form a pair (the half-split layout of the
    `apply_rotary_pos_emb` that the page's listing calls), i < rot_dim/2;
  * pair i turns by the angle p * theta_i at position p, with
    theta_i = base^(-2i / rot_dim) (base 10000 in the workloads):
        y_i          = x_i cos(p theta_i) - x_{i+h} sin(p theta_i)
        y_{i+h}      = x_{i+h} cos(p theta_i) + x_i sin(p theta_i);
  * the fused write rotates q and k in place (so a following prefill reads
    rotated rows) and stores the rotated k and the unrotated v into the pools
    exactly as ``kv_write`` does; stored values are the fp64 results rounded
    to the input dtype (nearest even).
"""
from __future__ import annotations

import numpy as np

from .attention import BF16, F32, kv_write, upcast


def inv_freq(rot_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i / rot_dim), i < rot_dim / 2, float64."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / rot_dim)


def cos_sin_table(max_positions: int, rot_dim: int, base: float) -> np.ndarray:
    """[max_positions, rot_dim] float64: cos(p theta_i) in the first half,
    sin(p theta_i) in the second."""
    ang = np.arange(max_positions, dtype=np.float64)[:, None] * inv_freq(rot_dim, base)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def rotate(x, positions, rot_dim: int, base: float, dtype: str) -> np.ndarray:
    """RoPE of rows x [T, H, d] (in `dtype`) at positions [T], float64."""
    x = upcast(x, dtype).copy()
    h = rot_dim // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(rot_dim, base)[None, :]   # [T, h]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., :h].copy()
    b = x[..., h:rot_dim].copy()
    x[..., :h] = a * c - b * s
    x[..., h:rot_dim] = b * c + a * s
    return x


def round_to(x64, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, nearest even (bf16 as uint16 bits).

    bf16 keeps 8 significant bits: with |x| = m 2^E, m in [0.5, 1), the
    neighbours are multiples of 2^(E-8); |x| / 2^(E-8) is exact in float64 and
    np.rint rounds it half to even.  (Finite inputs in bf16's normal range.)
    """
    f = np.asarray(x64, dtype=np.float64)
    if dtype == F32:
        return f.astype(np.float32)
    _, E = np.frexp(f)
    step = np.ldexp(1.0, E - 8)
    r = np.rint(f / step) * step                   # exact multiple, representable in fp32
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rope_kv_write(q, k, v, k_cache, v_cache, slot_mapping, positions, block_size, rot_dim, base, dtype):
    """The fused op: returns (q_rot, k_rot, k_cache', v_cache') with q_rot and
    k_rot in the input dtype (what the in-place rotation leaves in q and k)."""
    q_rot = round_to(rotate(q, positions, rot_dim, base, dtype), dtype)
    k_rot = round_to(rotate(k, positions, rot_dim, base, dtype), dtype)
    kc, vc = kv_write(k_cache, v_cache, k_rot, v, slot_mapping, block_size)
    return q_rot, k_rot, kc, vc
