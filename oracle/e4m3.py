"""OCP FP8 e4m3 ("e4m3fn") decoding (oracle; test infrastructure only).

The FP8 KV cache of the SGLang x HPC-Ops page ("Attention and MoE",
``--kv-cache-dtype fp8_e4m3``) stores e4m3 codes.  The OCP 8-bit floating
point format defines e4m3 as: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the all-ones
exponent with all-ones mantissa (0x7F, 0xFF) is NaN; there are no
infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np


def decode_code(code: int) -> float:
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 e4m3 codes to fp64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Values of e4m3 codes with one scale per row of the last axis:
    decode(codes) * scale[..., None], in fp64 (exact)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]
