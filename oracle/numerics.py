"""Storage formats used by the oracle: bf16, OCP fp8 e4m3 and symmetric int8.

Test infrastructure only: nothing on the product path may import this module.

Every conversion here is written from the published bit layout of the format,
not from any library routine, so that the tests can pin it against one:

* bf16 (bfloat16): 1 sign, 8 exponent, 7 mantissa bits; the upper half of an
  IEEE-754 binary32.  Narrowing is round-to-nearest-even on the 16 dropped bits.
* fp8 e4m3 as in the OCP 8-bit floating point specification ("E4M3FN"): 1 sign,
  4 exponent (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, the
  largest finite magnitude is 1.75 * 2**8 = 448, subnormals are m * 2**-9.
* int8: symmetric, codes -127..127, scale amax/127.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- bf16


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bit patterns must be uint16")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Narrow float32 to bf16 bit patterns, round to nearest, ties to even.

    Finite values beyond the largest bf16 round to +-inf like any other IEEE
    narrowing; NaN stays NaN (made quiet).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
    return r


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_to_f32(f32_to_bf16(x))


# ----------------------------------------------------------------------------- fp8 e4m3

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode e4m3 codes (uint8) to float32 (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = exp > 0
    mag = np.where(normal, (1.0 + man / 8.0) * np.exp2(exp - 7.0), man * 2.0 ** -9)
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return (sign * mag).astype(np.float32)


# The 127 non-negative finite magnitudes, code 0x00 .. 0x7E, increasing with the code.
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3 codes, round to nearest with ties to the even code, saturating.

    Nearest is taken over the 127 finite magnitudes; magnitudes at or above 448
    give 448.  NaN gives the NaN code.  Zero keeps its sign.
    """
    xf = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(xf)
    # index of the largest magnitude <= a
    lo = np.clip(np.searchsorted(_E4M3_POS, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(np.signbit(xf), 0x80, 0)
    code = np.where(np.isnan(xf), 0x7F, code)
    return code.astype(np.uint8)


def quant_e4m3_rows(x: np.ndarray, block: int = 128):
    """Per (row, block of `block` columns) dynamic e4m3 quantisation.

    amax is the largest magnitude in the block; the codes are e4m3(x * (448/amax))
    with the product and the quotient taken in float32, the scale is amax/448.
    An all-zero block gets codes 0 and scale 1.  Returns (codes, scales) with
    scales of shape (rows, cols/block).
    """
    x = np.asarray(x, dtype=np.float32)
    R, Cn = x.shape
    assert Cn % block == 0
    xb = x.reshape(R, Cn // block, block)
    amax = np.abs(xb).max(axis=2)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    inv = np.where(amax > 0, inv, np.float32(0.0)).astype(np.float32)
    q = e4m3_encode((xb * inv[:, :, None]).astype(np.float32))
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    return q.reshape(R, Cn), s.astype(np.float32)


def dequant_e4m3_rows(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    R, Cn = codes.shape
    v = e4m3_decode(codes).reshape(R, Cn // block, block)
    return (v * scales[:, :, None]).astype(np.float32).reshape(R, Cn)


def quant_e4m3_blocks(w: np.ndarray, block: int = 128):
    """Per (block x block) tile dynamic e4m3 quantisation of a 2-D matrix.

    Same rule as quant_e4m3_rows with the amax taken over the whole tile.
    Returns (codes, scales) with scales of shape (rows/block, cols/block).
    """
    w = np.asarray(w, dtype=np.float32)
    R, Cn = w.shape
    assert R % block == 0 and Cn % block == 0
    t = w.reshape(R // block, block, Cn // block, block)
    amax = np.abs(t).max(axis=(1, 3))
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, (np.float32(E4M3_MAX) / safe).astype(np.float32), np.float32(0.0))
    q = e4m3_encode((t * inv[:, None, :, None]).astype(np.float32)).reshape(R, Cn)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    return q, s.astype(np.float32)


def dequant_e4m3_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    R, Cn = codes.shape
    v = e4m3_decode(codes).reshape(R // block, block, Cn // block, block)
    return (v * scales[:, None, :, None]).astype(np.float32).reshape(R, Cn)


def quant_mx_e4m3_rows(x: np.ndarray, block: int = 32):
    """Microscaled (MX-style) e4m3 along rows: one E8M0 (power-of-two) scale per block
    of `block` consecutive values of a row.

    The scale X is the smallest power of two that brings the block maximum within the
    e4m3 range: amax / X <= 448, i.e. with amax = M * 2^E (1 <= M < 2), X = 2^(E - 8) when
    M <= 1.75 and 2^(E - 7) otherwise; it is clamped to the E8M0 range 2^-127 .. 2^127.
    Codes are e4m3(x / X), rounded to nearest even (no value saturates).  The scale byte
    is the exponent of X plus 127; an all-zero block gets byte 0 and codes 0.  Returns
    (codes (R, C) uint8, scales (R, C/block) uint8).
    """
    x = np.asarray(x, dtype=np.float32)
    R, Cn = x.shape
    assert Cn % block == 0
    xb = x.reshape(R, Cn // block, block).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    m, p = np.frexp(amax)                  # amax = m * 2^p, m in [0.5, 1): M = 2m, E = p - 1
    shared = np.where(amax > 0, (p - 1) - 8 + (m > 0.875), -127)
    shared = np.clip(shared, -127, 127)
    q = e4m3_encode((xb / np.exp2(shared)[:, :, None]).astype(np.float32))
    return q.reshape(R, Cn), (shared + 127).astype(np.uint8)


def dequant_mx_e4m3_rows(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """codes * 2^(scale byte - 127), float64 (exact)."""
    R, Cn = codes.shape
    v = e4m3_decode(codes).astype(np.float64).reshape(R, Cn // block, block)
    return (v * np.exp2(scales.astype(np.float64) - 127.0)[:, :, None]).reshape(R, Cn)


# ----------------------------------------------------------------------------- int8


def quant_int8_rows(x: np.ndarray):
    """Per-row symmetric int8: q = clamp(rint(x * (127/amax)), -127, 127), scale amax/127.

    rint rounds half to even; the product and quotient are float32.  An all-zero
    row gets codes 0 and scale 1.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, (np.float32(127.0) / safe).astype(np.float32), np.float32(0.0))
    q = np.clip(np.rint((x * inv[:, None]).astype(np.float32)), -127, 127).astype(np.int8)
    s = np.where(amax > 0, (amax / np.float32(127.0)).astype(np.float32), np.float32(1.0))
    return q, s.astype(np.float32)


def dequant_int8_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return (q.astype(np.float32) * s[:, None]).astype(np.float32)
