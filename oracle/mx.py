"""MXFP8 and MXFP4 weight quantisation of the oracle -- TEST INFRASTRUCTURE ONLY.

Written from the public OCP "Microscaling (MX) Formats Specification" v1.0:
  * section 5 (MX-compliant formats): an MX block is k = 32 elements that share
    one scale X; MXFP8 (E4M3) elements are OCP FP8 E4M3 numbers and X is an
    E8M0 number (an unsigned 8-bit exponent, value 2^(code - 127); code 255 is
    NaN);
  * section 5.3.3 (FP8 E4M3): exponent bias 7, 3 mantissa bits, subnormals,
    no infinities, S.1111.111 is NaN, largest normal 448, smallest normal 2^-6,
    smallest subnormal 2^-9;
  * section 6.3 (conversion from scalars): X = 2^(floor(log2(max_i |V_i|)) -
    emax_elem), emax_elem = 8 for E4M3 (the exponent of its largest normal
    power of two, 2^8), then each element is V_i / X rounded to the element
    format (round to nearest, ties to even); magnitudes above the largest
    normal saturate to it.
  * section 5.3.3 also defines MXFP4 (FP4 E2M1) elements: 1 sign, 2 exponent
    bits (bias 1), 1 mantissa bit, subnormal 0.5 at exponent 0, no infinity or
    NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. Its emax_elem is 2 (6 = 1.5 *
    2^2), so X = 2^(floor(log2 max|V|) - 2), and magnitudes above 6 saturate.
READING: the spec leaves X open for an all-zero block; the oracle uses the
smallest scale (code 0) and zero elements. The sign of an element that rounds
to zero is kept (0x80 for negative E4M3 inputs, 0x8 for E2M1).

The element rounding here is a plain nearest-value search over the non-negative
finite values of the element format, ties to the even code (for both formats
the even code is the one whose lowest mantissa bit is zero).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
EMAX_ELEM = 8
E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code (OCP MX spec v1.0, FP8 E4M3 element format)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = E4M3_TABLE[:127]          # codes 0..126: 0, subnormals, normals up to 448 (increasing)


def e8m0_value(code):
    """Shared-scale value 2^(code - 127) (code 255, NaN, never produced here)."""
    return np.ldexp(1.0, np.asarray(code, dtype=np.int64) - 127)


def round_e4m3(q) -> np.ndarray:
    """Codes of the E4M3 values nearest to q (ties to the even code), |q| > 448 saturating."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = np.abs(a - _POS[lo])
    d_hi = np.abs(_POS[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return mag | np.where(np.signbit(q), np.uint8(0x80), np.uint8(0)).astype(np.uint8)


def quantize_mxfp8(w):
    """Rows of w [N, K] (K a multiple of 32) -> (E4M3 codes uint8 [N, K], E8M0 scale codes uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - EMAX_ELEM, -127.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scale_codes = (e + 127).astype(np.uint8)
    q = blocks / np.ldexp(1.0, e)[..., None]
    codes = round_e4m3(q).reshape(n, k)
    return codes, scale_codes


def dequantize_mxfp8(codes, scale_codes) -> np.ndarray:
    """Element value times its block's scale, float64 [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    vals = E4M3_TABLE[codes].reshape(n, k // BLOCK, BLOCK)
    return (vals * e8m0_value(scale_codes)[..., None]).reshape(n, k)


# -------------------------------------------------------------------- MXFP4 (FP4 E2M1 elements)

EMAX_E2M1 = 2
E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of one FP4 E2M1 code (OCP MX spec v1.0): bias 1, exponent 0 is subnormal (m * 0.5)."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_POS4 = E2M1_TABLE[:8]           # codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (increasing)


def round_e2m1(q) -> np.ndarray:
    """Codes (0..15) of the E2M1 values nearest to q (ties to the even code), |q| > 6 saturating."""
    q = np.asarray(q, dtype=np.float64)
    a = np.minimum(np.abs(q), E2M1_MAX)
    hi = np.clip(np.searchsorted(_POS4, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_lo = np.abs(a - _POS4[lo])
    d_hi = np.abs(_POS4[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return mag | np.where(np.signbit(q), np.uint8(0x8), np.uint8(0)).astype(np.uint8)


def quantize_mxfp4(w):
    """Rows of w [N, K] (K a multiple of 32) -> (E2M1 codes uint8 [N, K], one per element, values
    0..15; E8M0 scale codes uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - EMAX_E2M1, -127.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scale_codes = (e + 127).astype(np.uint8)
    q = blocks / np.ldexp(1.0, e)[..., None]
    codes = round_e2m1(q).reshape(n, k)
    return codes, scale_codes


def dequantize_mxfp4(codes, scale_codes) -> np.ndarray:
    """Element value times its block's scale, float64 [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    vals = E2M1_TABLE[codes].reshape(n, k // BLOCK, BLOCK)
    return (vals * e8m0_value(scale_codes)[..., None]).reshape(n, k)
