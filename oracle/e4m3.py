"""OCP 8-bit floating point E4M3 ("fn" variant) codec, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format (OCP "OFP8" specification, E4M3 table): 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; no infinities; S.1111.111 (0x7F / 0xFF) is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448 (0x7E).  Exponent field 0 encodes
subnormals m/8 * 2^-6.  The source pages name exactly these NaN bytes as the
ones that poison a masked gather (sglang PR 39288, Root cause (1)) and quantise
with scale = amax / 448, i.e. to this format's largest finite value.

Encoding here is round-to-nearest-even with saturation to +-448 ("satfinite"),
keeping the sign of zero.  Input values are float64 numbers that are exactly
representable in float32 (the quantiser's input is a float32 quotient).
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9
NAN_CODES = (0x7F, 0xFF)


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(v: np.ndarray) -> np.ndarray:
    """float64 values (float32-representable) -> E4M3 codes, RNE, satfinite.

    NaN inputs give 0x7F with the input's sign bit (not used by the writer's
    tested paths)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)

    nan = np.isnan(a)
    sat = (~nan) & (a >= MAX_FINITE)
    sub = (~nan) & (a < MIN_NORMAL)
    nrm = (~nan) & (~sat) & (~sub)

    # subnormal range: multiples of 2^-9; a carry to 8 is the smallest normal (code 0x08)
    code[sub] = np.rint(a[sub] / SUBNORMAL_STEP).astype(np.int64)

    # normal range: exponent e = floor(log2 a) read exactly from frexp, step 2^(e-3)
    an = a[nrm]
    _, ex = np.frexp(an)            # an = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1
    q = np.rint(an / np.ldexp(1.0, e - 3)).astype(np.int64)   # in [8, 16]
    carry = q == 16
    e = e + carry
    q = np.where(carry, 8, q)
    c = ((e + 7) << 3) | (q - 8)
    code[nrm] = np.minimum(c, 0x7E)   # a value rounding past 448 saturates

    code[sat] = 0x7E
    code[nan] = 0x7F
    return (code.astype(np.uint8) | sign)
