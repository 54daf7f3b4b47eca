"""bfloat16 encode/decode written from the format definition (oracle, test infrastructure).

bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits (bias 127) and 7 stored fraction bits, so 8 significant bits for normal
numbers and a fixed quantum of 2**-133 for subnormals.  The pages name bf16 as
the tokenizer's default precision (Cosmos Tokenizer guide, sections 2 and 6;
Cosmos-Tokenize1-CV8x8x8-720p model card, "Software Integration").

``decode`` is exact (every bf16 value is a float64 value).  ``encode`` rounds a
float64 value straight to the nearest bf16 value, ties to even, with overflow
to infinity and NaN mapped to the canonical quiet NaN 0x7FC0.  It does not go
through float32, so there is no double rounding.
"""

import numpy as np

QNAN_BITS = 0x7FC0


def decode(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """float64 -> float64 holding the nearest bf16 value (ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    # |x| = m * 2**e with m in [0.5, 1): the leading bit has weight 2**(e-1).
    _, e = np.frexp(xf)
    # 8 significant bits for normals (leading exponent >= -126), else the
    # subnormal quantum 2**-133.
    q_exp = np.maximum(e, -125) - 8
    scaled = np.ldexp(xf, -q_exp)          # exact: scaling by a power of two
    rounded = np.ldexp(np.rint(scaled), q_exp)  # np.rint rounds half to even
    out[finite] = rounded
    return out


def encode(x):
    """float64 -> uint16 bf16 bit patterns, round to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    r = round_to_bf16(x)
    with np.errstate(over="ignore"):
        # every finite bf16 value is exactly a float32; values that rounded
        # past the largest bf16 become +-inf here, as RNE requires.
        r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(QNAN_BITS), bits)
    return bits.astype(np.uint16)


def ulp(x_bits):
    """Spacing of bf16 values at the given bf16 bit patterns (float64)."""
    v = np.abs(decode(x_bits))
    _, e = np.frexp(np.where(v == 0, 1.0, v))
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.where(v == 0, np.ldexp(1.0, -133), q)
