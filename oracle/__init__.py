"""CPU oracle for attention over a paged KV cache (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .attention import (  # noqa: F401
    BF16, F32, attend, decode, decode_partitions, gather,
    group_of, kv_write, num_partitions, paged_prefill, prefill, reduce_partitions, upcast,
    window_start, kv_rows,
)
from .e4m3 import E4M3, E4M3_MAX, E4M3_NAN, e4m3_encode, e4m3_value  # noqa: F401
from .fp8 import kv_write_fp8, quantize  # noqa: F401
from . import rope  # noqa: F401
