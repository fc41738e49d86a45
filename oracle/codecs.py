"""Storage number formats, built from their bit-field definitions.

[V4-vLLM] 2.1 (end) and 2.2 store the main KV in fp8 and the c4a indexer keys
in fp4; [vLLM-0.7.2] 2.2 names the fp8 flavour ``fp8_e4m3``.  The pages give no
bit layout, so the OCP definitions are used:

* E4M3 "FN": 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field
  0 is subnormal; no infinities; S.1111.111 is NaN, so the largest finite
  magnitude is 1.75 * 2**8 = 448.
* E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* bfloat16: the top 16 bits of an IEEE binary32.

Encoding rounds to nearest, ties to the even code, and saturates to the largest
finite magnitude; the sign is kept (so a value that rounds to zero keeps its
sign bit).  The tables below are generated from the field definitions, not
typed in.
"""

import numpy as np


def _e4m3_decode_scalar(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def _e2m1_decode_scalar(code: int) -> float:
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * (man / 2.0)
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


#: value of every E4M3 code (NaN at 0x7F and 0xFF), fp64
E4M3_TABLE = np.array([_e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
#: value of every E2M1 code (4-bit), fp64
E2M1_TABLE = np.array([_e2m1_decode_scalar(c) for c in range(16)], dtype=np.float64)

E4M3_MAX = float(E4M3_TABLE[0x7E])  # 448
E2M1_MAX = float(E2M1_TABLE[0x7])  # 6

# non-negative finite values in code order; both formats are monotone in the code
_E4M3_POS = E4M3_TABLE[:0x7F]
_E2M1_POS = E2M1_TABLE[:0x8]


def _encode_nearest_even(y, pos_values, max_value, sign_shift):
    """Round |y| to the nearest entry of ``pos_values`` (ascending, indexed by
    code), ties to the even code, saturating at ``max_value``; then add the
    sign bit at ``sign_shift``."""
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.int64)
    a = np.minimum(np.abs(y), max_value)
    hi = np.searchsorted(pos_values, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, len(pos_values) - 1)
    lo = np.clip(hi - 1, 0, len(pos_values) - 1)
    d_lo = a - pos_values[lo]
    d_hi = pos_values[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == pos_values[hi], hi, code)  # exact hits
    return (code | (sign << sign_shift)).astype(np.uint8)


def e4m3_encode(y):
    """fp32 value(s) -> E4M3 code(s) (uint8), RNE, saturating to +-448."""
    y32 = np.asarray(y, dtype=np.float32)
    return _encode_nearest_even(y32, _E4M3_POS, E4M3_MAX, 7)


def e4m3_decode(code):
    return E4M3_TABLE[np.asarray(code, dtype=np.int64)]


def e2m1_encode(y):
    """fp32 value(s) -> E2M1 code(s) (uint8 holding 4 bits), RNE, saturating to +-6."""
    y32 = np.asarray(y, dtype=np.float32)
    return _encode_nearest_even(y32, _E2M1_POS, E2M1_MAX, 3)


def e2m1_decode(code):
    return E2M1_TABLE[np.asarray(code, dtype=np.int64) & 0xF]


def bf16_encode(x):
    """fp32 -> bfloat16 bit pattern (uint16), round to nearest even.

    Adding 0x7FFF plus the lowest kept bit to the binary32 pattern carries into
    the kept half exactly when the dropped half is above one half ulp, or equal
    to it with an odd kept half; that is round-half-even.  Inputs are finite."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_decode(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
