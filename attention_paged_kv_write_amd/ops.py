"""ctypes binding over the C ABI of ``libpaged_attn.so`` (include/paged_attn.h).

Argument marshalling only: each function checks dtypes, shapes, contiguity and
device of torch tensors, allocates outputs the caller did not pass (torch is
the memory allocator), and hands raw device pointers plus the current HIP
stream to the C call of the same name.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  If the library is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

PA_F32, PA_BF16 = 0, 1
PA_OPT_FORCE_VECTOR_PATH = 1
EXPORTED_SYMBOLS = (
    "pa_abi_version", "pa_build_id", "pa_last_error", "pa_set_option", "paged_kv_write",
    "paged_attention_decode", "paged_attention_reduce", "varlen_causal_prefill",
    "paged_prefill", "paged_attention_decode_window", "varlen_causal_prefill_window",
    "paged_prefill_window", "paged_attention_reduce_window", "paged_kv_write_fp8",
    "paged_attention_decode_fp8", "rope_cos_sin_cache", "paged_kv_write_rope",
    "paged_attention_decode_append", "paged_attention_decode_append_fp8", "paged_kv_stream_read",
    "paged_attention_decode_noalloc", "pa_stream_read_contiguous",
)
PA_STREAM_LDS_DMA, PA_STREAM_REGISTERS = 0, 1
FP8_POOL_DTYPES = (torch.uint8, torch.float8_e4m3fn)   # E4M3 codes, one byte each

_lib: Optional[ctypes.CDLL] = None


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[code {code}] {message}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not found at {path}; build it with "
            "`python -m attention_paged_kv_write_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.pa_abi_version.restype = i32
    lib.pa_abi_version.argtypes = []
    lib.pa_build_id.restype = ctypes.c_char_p
    lib.pa_build_id.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_set_option.restype = i32
    lib.pa_set_option.argtypes = [i32, i32]
    lib.paged_kv_write.restype = i32
    lib.paged_kv_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.paged_attention_decode.restype = i32
    lib.paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                           f32, i32, vp]
    lib.paged_attention_reduce.restype = i32
    lib.paged_attention_reduce.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.varlen_causal_prefill.restype = i32
    lib.varlen_causal_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          f32, i32, vp]
    lib.paged_prefill.restype = i32
    lib.paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  i32, i32, i32, i32, f32, i32, vp]
    lib.paged_attention_decode_window.restype = i32
    lib.paged_attention_decode_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                  f32, i32, i32, vp]
    lib.varlen_causal_prefill_window.restype = i32
    lib.varlen_causal_prefill_window.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 f32, i32, i32, vp]
    lib.paged_kv_write_fp8.restype = i32
    lib.paged_kv_write_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp]
    lib.paged_attention_decode_fp8.restype = i32
    lib.paged_attention_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                               f32, vp, vp, i32, i32, vp]
    lib.paged_attention_decode_append.restype = i32
    lib.paged_attention_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                  f32, i32, i32, vp]
    lib.paged_attention_decode_append_fp8.restype = i32
    lib.paged_attention_decode_append_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                      i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                      f32, vp, vp, i32, i32, vp]
    lib.pa_stream_read_contiguous.restype = i32
    lib.pa_stream_read_contiguous.argtypes = [vp, vp, ctypes.c_uint64, i32, i32, vp]
    lib.rope_cos_sin_cache.restype = i32
    lib.rope_cos_sin_cache.argtypes = [vp, i32, i32, ctypes.c_double, vp]
    lib.paged_kv_write_rope.restype = i32
    lib.paged_kv_write_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                        i32, vp]
    lib.paged_attention_reduce_window.restype = i32
    lib.paged_attention_reduce_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.paged_prefill_window.restype = i32
    lib.paged_prefill_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, i32, i32, i32, f32, i32, i32, vp]
    lib.paged_attention_decode_noalloc.restype = i32
    lib.paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                   i32, i32, f32, i32, i32, vp]
    lib.paged_kv_stream_read.restype = i32
    lib.paged_kv_stream_read.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                         i32, vp]
    _lib = lib
    return lib


def build_id() -> str:
    """Source digest the loaded library was built from (pa_build_id)."""
    return load_library().pa_build_id().decode()


def check_build_id() -> str:
    """Raise unless the loaded library was built from the sources in this tree."""
    from .build import source_digest
    want, got = source_digest(), build_id()
    if got != want:
        raise RuntimeError(f"{LIB_PATH} was built from sources {got}, the tree holds {want}: rebuild it "
                           "(python -m attention_paged_kv_write_amd.build)")
    return got


def _check(rc: int) -> None:
    if rc != 0:
        msg = _lib.pa_last_error().decode() if _lib is not None else ""
        raise PagedAttnError(rc, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def set_force_vector_path(on: bool) -> None:
    """Route decode/prefill to the vector-ALU kernels (cross-checking aid)."""
    lib = load_library()
    _check(lib.pa_set_option(PA_OPT_FORCE_VECTOR_PATH, int(bool(on))))


def _scale_ptr(t: Optional[torch.Tensor], name: str) -> int:
    if t is None:
        raise ValueError(f"{name} is required for an FP8 (E4M3) pool")
    if t.numel() != 1:
        raise ValueError(f"{name} must hold one float32")
    return _dev(t, name, torch.float32)


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                   k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None) -> None:
    """Scatter k/v [T, H_kv, d] into the pools [NB, H_kv, bs, d] by slot (in place).
    Pools of uint8 / float8_e4m3fn hold E4M3 codes: k_scale / v_scale (one-element
    float32 device tensors) are then required and the rows are quantised."""
    lib = load_library()
    dt = _dtype_code(k)
    fp8 = k_cache.dtype in FP8_POOL_DTYPES
    for name, t in (("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        if fp8 and name != "v":
            if t.dtype != k_cache.dtype:
                raise TypeError(f"{name} dtype {t.dtype} != k_cache dtype {k_cache.dtype}")
        elif t.dtype != k.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != k dtype {k.dtype}")
    pk = _dev(k, "k", ndim=3)
    pv = _dev(v, "v", ndim=3)
    pkc = _dev(k_cache, "k_cache", ndim=4)
    pvc = _dev(v_cache, "v_cache", ndim=4)
    ps = _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    T, H, d = k.shape
    NB, H2, bs, d2 = k_cache.shape
    if v.shape != k.shape or v_cache.shape != k_cache.shape or H2 != H or d2 != d:
        raise ValueError("paged_kv_write: inconsistent shapes")
    if slot_mapping.shape[0] != T:
        raise ValueError("paged_kv_write: slot_mapping length != num_tokens")
    if fp8:
        _check(lib.paged_kv_write_fp8(pk, pv, pkc, pvc, ps, T, H, d, bs, NB, _scale_ptr(k_scale, "k_scale"),
                                      _scale_ptr(v_scale, "v_scale"), dt, _stream(k)))
        return
    _check(lib.paged_kv_write(pk, pv, pkc, pvc, ps, T, H, d, bs, NB, dt, _stream(k)))


def rope_cos_sin_cache(max_positions: int, rot_dim: int, base: float = 10000.0,
                       device: Optional[torch.device] = None) -> torch.Tensor:
    """The RoPE table [max_positions, rot_dim] float32 (cos then sin per row)."""
    lib = load_library()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    table = torch.empty((max_positions, rot_dim), dtype=torch.float32, device=dev)
    _check(lib.rope_cos_sin_cache(table.data_ptr() if table.numel() else None, int(max_positions), int(rot_dim),
                                  float(base), torch.cuda.current_stream(dev).cuda_stream))
    return table


def paged_kv_write_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, slot_mapping: torch.Tensor, positions: torch.Tensor,
                        cos_sin: torch.Tensor) -> None:
    """Rotate q [T,H_q,d] and k [T,H_kv,d] in place at `positions` with the table
    `cos_sin` [max_positions, rot_dim], and write rotated k and v into the pools."""
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    T, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if k.shape != (T, Hkv, d) or v.shape != k.shape or v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("paged_kv_write_rope: inconsistent shapes")
    if slot_mapping.shape != (T,) or positions.shape != (T,):
        raise ValueError("paged_kv_write_rope: slot_mapping / positions length != num_tokens")
    if cos_sin.dim() != 2:
        raise ValueError("paged_kv_write_rope: cos_sin must be [max_positions, rot_dim]")
    P, rot = cos_sin.shape
    _check(lib.paged_kv_write_rope(_dev(q, "q", ndim=3), _dev(k, "k", ndim=3), _dev(v, "v", ndim=3),
                                   _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
                                   _dev(slot_mapping, "slot_mapping", torch.int32, 1),
                                   _dev(positions, "positions", torch.int32, 1),
                                   _dev(cos_sin, "cos_sin", torch.float32, 2),
                                   T, Hq, Hkv, d, rot, bs, NB, P, dt, _stream(q)))


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return max(1, -(-int(max_context_len) // int(partition_size)))


def paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float,
                           partition_size: int = 0, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           part_out: Optional[torch.Tensor] = None,
                           part_lse: Optional[torch.Tensor] = None, window: int = 0,
                           k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                           k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None
                           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """PagedAttention decode.  Returns (out, lse), or (part_out, part_lse) when split.
    window > 0 keeps only the last `window` positions (sliding window).  Pools of
    uint8 / float8_e4m3fn hold E4M3 codes read with k_scale / v_scale.  k_new /
    v_new [B, H_kv, d]: the token at position ctx-1 of each sequence, stored into
    the pools by the same launch before it is read (the step's cache write)."""
    lib = load_library()
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    fp8 = k_cache.dtype in FP8_POOL_DTYPES
    kv_dtype_ok = (v_cache.dtype == k_cache.dtype) and (fp8 or k_cache.dtype == q.dtype)
    if d2 != d or v_cache.shape != k_cache.shape or not kv_dtype_ok:
        raise ValueError("paged_attention_decode: inconsistent q / cache shapes or dtypes")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_attention_decode: block_tables / context_lens shape")
    pq = _dev(q, "q", ndim=3)
    pkc = _dev(k_cache, "k_cache", ndim=4)
    pvc = _dev(v_cache, "v_cache", ndim=4)
    pbt = _dev(block_tables, "block_tables", torch.int32, 2)
    pcl = _dev(context_lens, "context_lens", torch.int32, 1)
    po = pl = ppo = ppl = None
    if partition_size > 0:
        P = num_partitions(max_context_len, partition_size)
        if part_out is None:
            part_out = torch.empty((B, Hq, P, d), dtype=torch.float32, device=q.device)
        if part_lse is None:
            part_lse = torch.empty((B, Hq, P), dtype=torch.float32, device=q.device)
        if part_out.shape != (B, Hq, P, d) or part_lse.shape != (B, Hq, P):
            raise ValueError("paged_attention_decode: part_out/part_lse shape")
        ppo = _dev(part_out, "part_out", torch.float32)
        ppl = _dev(part_lse, "part_lse", torch.float32)
    else:
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        if out.shape != q.shape or lse.shape != (B, Hq):
            raise ValueError("paged_attention_decode: out/lse shape")
        po = _dev(out, "out", q.dtype)
        pl = _dev(lse, "lse", torch.float32)
    if (k_new is None) != (v_new is None):
        raise ValueError("paged_attention_decode: give both k_new and v_new, or neither")
    if k_new is not None:
        if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape or k_new.dtype != q.dtype or \
                v_new.dtype != q.dtype:
            raise ValueError("paged_attention_decode: k_new / v_new must be [B, H_kv, d] in q's dtype")
        pkn, pvn = _dev(k_new, "k_new", ndim=3), _dev(v_new, "v_new", ndim=3)
        if fp8:
            _check(lib.paged_attention_decode_append_fp8(
                po, pl, ppo, ppl, pq, pkn, pvn, pkc, pvc, pbt, pcl, B, Hq, Hkv, d, bs, block_tables.shape[1], NB,
                int(partition_size), int(max_context_len), float(scale), _scale_ptr(k_scale, "k_scale"),
                _scale_ptr(v_scale, "v_scale"), int(window), dt, _stream(q)))
        else:
            _check(lib.paged_attention_decode_append(
                po, pl, ppo, ppl, pq, pkn, pvn, pkc, pvc, pbt, pcl, B, Hq, Hkv, d, bs, block_tables.shape[1], NB,
                int(partition_size), int(max_context_len), float(scale), int(window), dt, _stream(q)))
    elif fp8:
        _check(lib.paged_attention_decode_fp8(po, pl, ppo, ppl, pq, pkc, pvc, pbt, pcl, B, Hq, Hkv, d, bs,
                                              block_tables.shape[1], NB, int(partition_size),
                                              int(max_context_len), float(scale), _scale_ptr(k_scale, "k_scale"),
                                              _scale_ptr(v_scale, "v_scale"), int(window), dt, _stream(q)))
    else:
        _check(lib.paged_attention_decode_window(po, pl, ppo, ppl, pq, pkc, pvc, pbt, pcl, B, Hq, Hkv, d, bs,
                                                 block_tables.shape[1], NB, int(partition_size),
                                                 int(max_context_len), float(scale), int(window), dt,
                                                 _stream(q)))
    if partition_size > 0:
        return part_out, part_lse
    return out, lse


def paged_attention_reduce(part_out: torch.Tensor, part_lse: torch.Tensor,
                           context_lens: torch.Tensor, partition_size: int,
                           out_dtype: torch.dtype = torch.bfloat16,
                           out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Log-sum-exp merge of split-KV partitions -> (out [B, H_q, d], lse [B, H_q]).
    window: the sliding window the partitions were computed with (the merge
    starts at the partition holding the window's first key)."""
    lib = load_library()
    B, Hq, P, d = part_out.shape
    if part_lse.shape != (B, Hq, P) or context_lens.shape != (B,):
        raise ValueError("paged_attention_reduce: shapes")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=part_out.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=part_out.device)
    if out.shape != (B, Hq, d) or lse.shape != (B, Hq):
        raise ValueError("paged_attention_reduce: out must be [B, H_q, d] and lse [B, H_q]")
    dt = _dtype_code(out)
    _check(lib.paged_attention_reduce_window(_dev(out, "out", ndim=3), _dev(lse, "lse", torch.float32, 2),
                                             _dev(part_out, "part_out", torch.float32, 4),
                                             _dev(part_lse, "part_lse", torch.float32, 3),
                                             _dev(context_lens, "context_lens", torch.int32, 1),
                                             B, Hq, d, int(partition_size), P, int(window), dt,
                                             _stream(part_out)))
    return out, lse


def varlen_causal_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          cu_seqlens: torch.Tensor, max_seqlen: int,
                          scale: float, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Causal attention over sequences packed by cu_seqlens -> (out [T,H_q,d], lse [T,H_q]).
    window > 0 keeps only the last `window` keys of each row (sliding window)."""
    lib = load_library()
    dt = _dtype_code(q)
    T, Hq, d = q.shape
    T2, Hkv, d2 = k.shape
    if T2 != T or d2 != d or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("varlen_causal_prefill: inconsistent q/k/v")
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("varlen_causal_prefill: cu_seqlens must be [num_seqs + 1]")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or lse.shape != (T, Hq):
        raise ValueError("varlen_causal_prefill: out must be [T, H_q, d] and lse [T, H_q]")
    _check(lib.varlen_causal_prefill_window(_dev(out, "out", q.dtype, 3), _dev(lse, "lse", torch.float32, 2),
                                            _dev(q, "q", ndim=3), _dev(k, "k", ndim=3), _dev(v, "v", ndim=3),
                                            _dev(cu_seqlens, "cu_seqlens", torch.int32, 1),
                                            cu_seqlens.shape[0] - 1, T, int(max_seqlen), Hq, Hkv, d,
                                            float(scale), int(window), dt, _stream(q)))
    return out, lse


def paged_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor, context_lens: torch.Tensor,
                  max_seqlen_q: int, max_context_len: int, scale: float,
                  out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """A chunk of query rows per sequence (the last rows of its cache) against its
    paged cache -> (out [T_q,H_q,d], lse [T_q,H_q]); window > 0: sliding window."""
    lib = load_library()
    dt = _dtype_code(q)
    T, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("paged_prefill: inconsistent q / cache shapes or dtypes")
    S = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_q.dim() != 1 or S < 0 or block_tables.dim() != 2 or block_tables.shape[0] != S \
            or context_lens.shape != (S,):
        raise ValueError("paged_prefill: cu_seqlens_q / block_tables / context_lens shape")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or lse.shape != (T, Hq):
        raise ValueError("paged_prefill: out must be [T_q, H_q, d] and lse [T_q, H_q]")
    _check(lib.paged_prefill_window(_dev(out, "out", q.dtype, 3), _dev(lse, "lse", torch.float32, 2),
                             _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", ndim=4),
                             _dev(v_cache, "v_cache", ndim=4),
                             _dev(block_tables, "block_tables", torch.int32, 2),
                             _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1),
                             _dev(context_lens, "context_lens", torch.int32, 1),
                             S, T, int(max_seqlen_q), Hq, Hkv, d, bs, block_tables.shape[1], NB,
                             int(max_context_len), float(scale), int(window), dt, _stream(q)))
    return out, lse


def paged_kv_stream_read(k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, max_context_len: int, partition_size: int,
                         mode: int = PA_STREAM_LDS_DMA, depth: int = 2,
                         checksums: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Measurement call: read every K/V row a split decode with this partition
    size reads, in its work units and tiles, and return the XOR of their 32-bit
    words per (sequence, KV head, partition) as int32 [B, H_kv, P] (bit patterns)."""
    lib = load_library()
    NB, Hkv, bs, d = k_cache.shape
    B = context_lens.shape[0]
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or block_tables.dim() != 2 \
            or block_tables.shape[0] != B:
        raise ValueError("paged_kv_stream_read: inconsistent shapes")
    P = num_partitions(max_context_len, partition_size)
    if checksums is None:
        checksums = torch.empty((B, Hkv, P), dtype=torch.int32, device=k_cache.device)
    if checksums.shape != (B, Hkv, P):
        raise ValueError("paged_kv_stream_read: checksums must be [B, H_kv, P]")
    _check(lib.paged_kv_stream_read(_dev(checksums, "checksums", torch.int32, 3), _dev(k_cache, "k_cache", ndim=4),
                                    _dev(v_cache, "v_cache", ndim=4),
                                    _dev(block_tables, "block_tables", torch.int32, 2),
                                    _dev(context_lens, "context_lens", torch.int32, 1), B, Hkv, d, bs,
                                    block_tables.shape[1], NB, int(partition_size), int(max_context_len), int(mode),
                                    int(depth), _dtype_code(k_cache), _stream(k_cache)))
    return checksums


def stream_read_contiguous(src: torch.Tensor, waves: int = 2048, depth: int = 4,
                           checksums: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The plain read ceiling: every byte of the (contiguous) device tensor src
    read front to back in 16-byte non-temporal loads, wave w taking an equal
    contiguous share; returns the per-wave XOR checksums (uint32 viewed as
    int32 [waves])."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if nbytes % 16:
        raise ValueError("stream_read_contiguous: the tensor's size must be a multiple of 16 bytes")
    if checksums is None:
        checksums = torch.empty((waves,), dtype=torch.int32, device=src.device)
    if checksums.shape != (waves,):
        raise ValueError("stream_read_contiguous: checksums must be [waves]")
    _check(lib.pa_stream_read_contiguous(_dev(checksums, "checksums", torch.int32, 1), _dev(src, "src"),
                                         nbytes, int(waves), int(depth), _stream(src)))
    return checksums

def paged_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                                   scale: float, partition_size: int, out: torch.Tensor, lse: torch.Tensor,
                                   window: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split decode and its merge in one library call that allocates nothing:
    the partials live in the library's per-GPU scratch (at most 32 MiB of
    them), so the caller passes only inputs and the outputs out [B, H_q, d]
    and lse [B, H_q].  Calls that overlap on one GPU race on that scratch."""
    lib = load_library()
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("paged_attention_decode_noalloc: inconsistent q / cache shapes or dtypes")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("paged_attention_decode_noalloc: block_tables / context_lens shape")
    if out.shape != q.shape or lse.shape != (B, Hq):
        raise ValueError("paged_attention_decode_noalloc: out must be [B, H_q, d] and lse [B, H_q]")
    _check(lib.paged_attention_decode_noalloc(
        _dev(out, "out", q.dtype, 3), _dev(lse, "lse", torch.float32, 2), _dev(q, "q", ndim=3),
        _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
        B, Hq, Hkv, d, bs, block_tables.shape[1], NB, int(partition_size), int(max_context_len), float(scale),
        int(window), dt, _stream(q)))
    return out, lse
