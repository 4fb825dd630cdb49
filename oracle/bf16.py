"""bfloat16 as a number format, written from its definition.

bfloat16 keeps the sign and the 8-bit exponent of IEEE binary32 and 7 stored
fraction bits, so a finite value has 8 significant bits; normal numbers span
exponents -126..127 and subnormals are spaced 2**-133 apart. Rounding is to
nearest, ties to even. The pages fix BF16 as the compute and storage type
("Hy-Nomas: Towards Free-Form Interactive World Generation", section
"Single-GPU Low-Memory Inference": INT8 storage while attention stays BF16).

Bit patterns are carried as numpy uint16 arrays.
"""

import numpy as np

_MIN_QUANTUM_EXP = -133   # spacing of bf16 subnormals: 2**-126 * 2**-7


def bf16_bits_to_f64(bits):
    """Exact value of each bf16 bit pattern as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    Written as the definition: with |x| = m * 2**e (0.5 <= m < 1), the bf16
    grid around x has spacing 2**(e - 8), but never finer than 2**-133.
    Dividing by a power of two is exact in float64 and ``np.rint`` rounds
    half to even, so ``rint(x / q) * q`` is the correctly rounded value.
    Values at or beyond the bf16 overflow threshold become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    _, e = np.frexp(x[fin])
    q = np.maximum(e - 8, _MIN_QUANTUM_EXP)
    r = np.rint(np.ldexp(x[fin], -q))
    y = np.ldexp(r, q)
    # largest finite bf16 is (2 - 2**-7) * 2**127; anything that rounds past it
    # is an overflow
    big = np.abs(y) >= 2.0 ** 128
    y[big] = np.copysign(np.inf, y[big])
    out[fin] = y
    return out


def f64_to_bf16_bits(x):
    """Round to bf16 (ties to even) and return the bit patterns as uint16."""
    y = round_to_bf16(x)
    # y has at most 8 significant bits, so the float32 conversion is exact and
    # its low 16 bits are zero.
    b = y.astype(np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)
