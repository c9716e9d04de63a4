"""Element and scale formats, written out from their definitions (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The sources name the formats only as "MXFP4 expert weights" and "online FP8
activations" ("Pushing the Limits of Serving DeepSeek-V4-Pro", §2.2). The
definitions are the OCP ones:

* E2M1 (MXFP4 element): bits S EE M, exponent bias 1. E = 0 is subnormal,
  value M * 0.5; otherwise (1 + M/2) * 2^(E-1). Magnitudes 0, .5, 1, 1.5, 2, 3,
  4, 6. No Inf, no NaN. Two codes per byte; the low nibble is the element with
  the even index along K.
* E8M0 (MX scale): value 2^(c - 127); c = 255 is NaN.
* E4M3FN (OCP FP8): bits S EEEE MMM, bias 7. E = 0 is subnormal, value
  (M/8) * 2^-6; otherwise (1 + M/8) * 2^(E-7). S.1111.111 is NaN; no Inf.
  Largest finite 448, smallest subnormal 2^-9.

Reading taken where the pages are silent: activation blocks are 128 columns of
one token, each with a power-of-two (E8M0) scale chosen as the smallest 2^e
with amax <= 448 * 2^e, and elements are rounded to nearest, ties to even, on
the E4M3 grid of x / 2^e. Because the scale is a power of two the division is
exact, and because it is the smallest one that fits, no element saturates.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * m * 0.5
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: E2M1 code (0..15) -> float64 value
E2M1_VALUES = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
#: E4M3FN code (0..255) -> float64 value (NaN for 0x7F / 0xFF)
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
#: E8M0 code (0..255) -> float64 value (NaN for 255)
E8M0_VALUES = np.array([2.0 ** (c - 127) if c != 255 else np.nan for c in range(256)],
                       dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even (finite
    inputs within the bf16 range). Rounds once, straight from float64: normal
    bf16 numbers have 8 significant bits (spacing 2^(p-7) in [2^p, 2^(p+1))),
    subnormals a fixed spacing of 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                    # a = m * 2^ex, m in [0.5, 1)
    step_exp = np.where(a >= 2.0 ** -126, ex - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(a, -step_exp)), step_exp)
    u = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact
    return np.where(np.signbit(v), u | np.uint16(0x8000), u).astype(np.uint16)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float64 values to E4M3FN codes: nearest, ties to even, saturating
    at +-448, sign kept (negative values that round to zero give 0x80).

    The grid spacing for |v| in [2^p, 2^(p+1)) with p >= -6 is 2^(p-3); below
    2^-6 (subnormals) it is 2^-9. Rounding |v| / spacing to the nearest integer
    with ties to even is exact in float64 (the spacing is a power of two).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                    # a = m * 2^ex, m in [0.5, 1) -> p = ex - 1
    step_exp = np.where(a >= 2.0 ** -6, ex - 1 - 3, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -step_exp)), step_exp)
    r = np.minimum(r, E4M3_MAX)
    # code from the rounded magnitude (which may have moved up a binade)
    _, rex = np.frexp(r)
    normal = r >= 2.0 ** -6
    E = np.where(normal, rex - 1 + 7, 0)
    M = np.where(normal, np.ldexp(r, -(rex - 1)) * 8 - 8, np.ldexp(r, 9))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    code = np.where(r == 0, 0, code)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Power-of-two block scale exponent: the smallest integer e with
    amax <= 448 * 2^e, clamped to the E8M0 range [-127, 127].

    With amax = m * 2^p, m in [1, 2): 448 = 1.75 * 2^8, so e = p - 8 when
    m <= 1.75 and e = p - 7 otherwise. amax = 0 gives the smallest scale, -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)                 # amax = (2m) * 2^(ex-1), 2m in [1, 2)
    p = ex - 1
    e = np.where(2.0 * m <= 1.75, p - 8, p - 7)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_blocks(v: np.ndarray, block: int = 128):
    """Quantize rows of float64 values to E4M3 codes with one E8M0 scale per
    ``block`` consecutive columns. Returns (codes uint8 [R, C], scale codes uint8
    [R, C/block], amax float64 [R, C/block])."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    assert C % block == 0
    vb = v.reshape(R, C // block, block)
    amax = np.abs(vb).max(axis=-1)
    e = scale_exponent(amax)
    codes = e4m3_encode(np.ldexp(vb, -e[..., None]))
    return codes.reshape(R, C), (e + 127).astype(np.uint8), amax


def dequantize_blocks(codes: np.ndarray, scale_codes: np.ndarray, block: int = 128) -> np.ndarray:
    """Inverse of quantize_blocks: E4M3 value * 2^(scale - 127), exact in float64."""
    R, C = codes.shape
    vals = E4M3_VALUES[codes].reshape(R, C // block, block)
    return (vals * E8M0_VALUES[scale_codes][..., None]).reshape(R, C)
