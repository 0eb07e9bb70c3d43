"""fp64 CPU oracle for an FP8 (E4M3) paged KV cache.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it.  It shares no code with the HIP path.

The pages enable KV-cache quantisation and speak of FP8 with dynamic scaling
("Llama 4 inference doubling (FlashAttention-3 + PagedAttention + vLLM)",
chapter 1 on grouped-query attention with FP8, and section 3.2's
`enable_kv_cache_quantization` switch) but fix neither the FP8 encoding nor
the scale's granularity.  Readings taken here:
  * the encoding is OCP FP8 E4M3 (the E4M3 of the OCP 8-bit floating point
    specification): sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals at exponent field 0, no infinities, S.1111.111 is NaN; the
    largest finite magnitude is 448;
  * one scale per K pool and one per V pool (fp32, chosen by the caller, who
    may compute it from the data: that is the dynamic part); a value x is
    stored as the code nearest to x / scale and read back as code * scale;
  * x / scale is one IEEE fp32 division of the fp32 value (bf16 inputs are
    widened exactly first); the code is the nearest E4M3 value to that fp32
    quotient, ties to the even code (mantissa LSB 0); magnitudes at or past
    448 saturate to +-448; NaN gives code 0x7F;
  * attention over such a cache is the plain attention of the dequantised
    K and V (code value times scale, exact in fp64).
"""
from __future__ import annotations

import numpy as np

from .attention import upcast
from .e4m3 import E4M3, E4M3_MAX, E4M3_NAN, e4m3_encode, e4m3_value  # noqa: F401


def quantize(x, dtype, scale) -> np.ndarray:
    """Codes of x (in `dtype`, widened exactly) divided by `scale` in fp32."""
    q = upcast(x, dtype).astype(np.float32) / np.float32(scale)
    return e4m3_encode(q)


def kv_write_fp8(k_cache, v_cache, k, v, slot_mapping, block_size, dtype, k_scale, v_scale):
    """The cache write of ``attention.kv_write`` into E4M3 pools: token t with
    slot s >= 0 stores quantize(k[t]) and quantize(v[t]) at block s // bs,
    offset s % bs of every KV head; a negative slot is skipped."""
    kc = np.array(k_cache, dtype=np.uint8, copy=True)
    vc = np.array(v_cache, dtype=np.uint8, copy=True)
    kq = quantize(k, dtype, k_scale)
    vq = quantize(v, dtype, v_scale)
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        kc[blk, :, off, :] = kq[t]
        vc[blk, :, off, :] = vq[t]
    return kc, vc
