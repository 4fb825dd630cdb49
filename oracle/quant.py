"""Symmetric per-token, per-head INT8 quantisation of cached K and V.

Source: "Hy-Nomas: Towards Free-Form Interactive World Generation", section
"Single-GPU Low-Memory Inference" (cached keys and values are stored in INT8
while attention is computed in BF16); "Tencent Opens Hy-Nomas ...", section
"How the RTX 4090 configuration saves memory" (INT8 KV cache, BF16 attention).
The pages do not give the quantiser; the scheme taken here is:

* one fp32 scale per (token, head) over its 128 values:
  scale = fp32(absmax / 127), IEEE fp32 division;
* code = clamp(round_half_even(fp32(x / scale)), -127, 127), IEEE fp32 division;
* a token-head whose values are all zero gets scale 0 and all-zero codes;
* dequantised value = code * scale; where attention runs in BF16 the value
  fed to it is bf16(fp32(code * scale)): the exact product rounded to fp32,
  then to bf16, both round-to-nearest-even (the reading taken here).

Emulating fp32 division: both operands are fp32 values, so the float64
quotient rounded to fp32 equals the IEEE fp32 quotient (float64 carries
53 >= 2*24 + 2 bits, which makes the double rounding innocuous for division).
"""

import numpy as np

from .bf16 import round_to_bf16


def quantise_int8(x):
    """x: float64 [..., D] holding bf16 (hence fp32-exact) values.

    Returns (codes int8 [..., D], scales float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(x == x.astype(np.float32)):
        raise ValueError("inputs must be fp32-representable")
    a = np.max(np.abs(x), axis=-1)                                # exact
    scale = (a / 127.0).astype(np.float32)                        # IEEE fp32 a/127
    s64 = scale.astype(np.float64)[..., None]
    nz = s64 != 0.0
    q = np.where(nz, x / np.where(nz, s64, 1.0), 0.0)
    q = q.astype(np.float32).astype(np.float64)                   # IEEE fp32 x/scale
    codes = np.clip(np.rint(q), -127.0, 127.0)
    return codes.astype(np.int8), scale


def dequantise_int8(codes, scales):
    """code * scale, exact in float64."""
    return (np.asarray(codes, dtype=np.float64)
            * np.asarray(scales, dtype=np.float64)[..., None])


def dequantise_int8_bf16(codes, scales):
    """bf16(fp32(code * scale)) as float64: the BF16 operand attention uses.

    code * scale is exact in float64 (7 + 24 significant bits); astype(float32)
    rounds it to nearest even, and round_to_bf16 rounds that to bf16.
    """
    exact = dequantise_int8(codes, scales)
    return round_to_bf16(exact.astype(np.float32).astype(np.float64))
