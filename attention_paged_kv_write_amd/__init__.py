"""Attention over a paged KV cache, native to MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/paged_attn.h``).  ``ops`` is a thin ctypes
binding over it: it marshals torch tensors (device memory and the current
stream) into the C calls and does nothing else.
"""
__all__ = ["paged_kv_write", "paged_attention_decode", "paged_attention_reduce",
           "varlen_causal_prefill"]


def __getattr__(name):
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
