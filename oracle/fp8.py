"""fp64 decoder of 8-bit floating-point E4M3 codes (the OCP 8-bit
floating point format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; no infinities; exponent and mantissa all ones is NaN).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it.

"Context Window Scaling: YaRN, LongRoPE, and RingAttention Architectures"
(tecvarsity), Section 7, FAQ 3, names quantising the KV cache to FP8 but
fixes no format; E4M3 is the reading taken (the format gfx950's conversion
instructions decode), written out here from the format's definition.
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte code, exactly, in float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * np.exp2(1.0 - 7.0)
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)
