"""Brute-force per-token, per-expert statement of the FFN, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written independently of ``formats`` / ``moe`` so that the two can pin each
other: element values come from exact fractions built from the bit fields,
E4M3 rounding is a nearest-point search over every finite code (ties to the
code with an even mantissa), the block scale is found by searching exponents
upward until the block fits under 448, bf16 rounding is a binary search over the
ordered positive bit patterns with exact comparisons, dot products are
``math.fsum`` over exact products, and everything loops token by token and pick
by pick.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

_E4M3_MAX = Fraction(448)


def e2m1(code: int) -> Fraction:
    sign = -1 if (code >> 3) & 1 else 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        return sign * Fraction(man, 2)
    return sign * (1 + Fraction(man, 2)) * Fraction(2) ** (exp - 1)


def e4m3(code: int) -> Fraction:
    sign = -1 if (code >> 7) & 1 else 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 0:
        return sign * Fraction(man, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(man, 8)) * Fraction(2) ** (exp - 7)


_POS_CODES = [c for c in range(0x7F)]          # 0x00..0x7E: every finite non-negative code
_POS_VALUES = [e4m3(c) for c in _POS_CODES]


def e4m3_nearest(v: Fraction, negative: bool = None) -> int:
    """Nearest finite E4M3 code to v; ties go to the even mantissa; |v| > 448
    saturates; a negative v keeps its sign bit even when it rounds to zero
    (``negative`` carries the sign of a float -0.0, which a Fraction cannot)."""
    if negative is None:
        negative = v < 0
    a = abs(v)
    if a >= _E4M3_MAX:
        best = 0x7E
    else:
        best, bestd = None, None
        for c, val in zip(_POS_CODES, _POS_VALUES):
            d = abs(val - a)
            if bestd is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
                best, bestd = c, d
    return best | (0x80 if negative else 0)


_BF16_MAX_FINITE = 0x7F7F


def bf16_nearest(v: float) -> int:
    """Nearest bf16 bit pattern to the float v (finite, within range); ties go
    to the even pattern; the sign bit follows v's (also for -0.0 and values that
    round to zero). Positive bf16 patterns 0 .. 0x7F7F increase with their value,
    so the largest pattern at or below |v| is found by bisection."""
    a = abs(Fraction(v))
    lo, hi = 0, _BF16_MAX_FINITE
    while lo < hi:                      # largest pattern with value <= a
        mid = (lo + hi + 1) // 2
        if bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    best = lo
    if lo < _BF16_MAX_FINITE:
        d0 = a - bf16_value(lo)
        d1 = bf16_value(lo + 1) - a
        if d1 < d0 or (d1 == d0 and (lo & 1) == 1):
            best = lo + 1
    return best | (0x8000 if math.copysign(1.0, v) < 0 else 0)


def block_scale(amax: Fraction) -> int:
    """Smallest e in [-127, 127] with amax <= 448 * 2^e."""
    e = -127
    while e < 127 and amax > _E4M3_MAX * Fraction(2) ** e:
        e += 1
    return e


def quant_block(vals):
    """vals: list of floats (one block) -> (codes, e)."""
    amax = max(abs(Fraction(v)) for v in vals)
    e = block_scale(amax)
    s = Fraction(2) ** e
    return [e4m3_nearest(Fraction(v) / s, math.copysign(1.0, v) < 0) for v in vals], e


def bf16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


def mxfp4_row(codes_row, scales_row):
    """Packed MXFP4 row -> list of Fractions."""
    out = []
    for byte in codes_row:
        for nib in (int(byte) & 15, int(byte) >> 4):
            k = len(out)
            out.append(e2m1(nib) * Fraction(2) ** (int(scales_row[k // 32]) - 127))
    return out


def nvfp4_row(codes_row, scales_row, tensor_scale):
    """Packed NVFP4 row (E4M3 scale per 16) times the tensor scale -> Fractions."""
    out = []
    gs = Fraction(float(tensor_scale))
    for byte in codes_row:
        for nib in (int(byte) & 15, int(byte) >> 4):
            k = len(out)
            out.append(e2m1(nib) * e4m3(int(scales_row[k // 16])) * gs)
    return out


def fp8_block_row(codes_row, scales_grid, n: int):
    """FP8 weight row n with 128x128 block scales -> list of Fractions."""
    return [e4m3(int(c)) * Fraction(2) ** (int(scales_grid[n // 128][k // 128]) - 127)
            for k, c in enumerate(codes_row)]


def _dot(a, b) -> float:
    # a, b hold floats that are exact binary values with few significant bits:
    # every product is exact in float64, and fsum rounds the exact sum once
    return math.fsum(x * y for x, y in zip(a, b))


def _floats(rows):
    return [[float(v) for v in r] for r in rows]


def _quantize_dequant(vec, block=128):
    out, codes, scales = [], [], []
    for b0 in range(0, len(vec), block):
        c, e = quant_block([float(v) for v in vec[b0:b0 + block]])
        codes += c
        scales.append(e + 127)
        out += [float(e4m3(ci) * Fraction(2) ** e) for ci in c]
    return out, codes, scales


def _expert(xh, rows13, rows2, I, act="fp8"):
    acc = [_dot(r, xh) for r in rows13]
    h = []
    for n in range(I):
        g, u = acc[n], acc[I + n]
        # exp(-g) overflows below about -709: silu(g) is then -0.0 (g / inf)
        h.append((g / (1.0 + math.exp(-g)) if g > -700 else g * 0.0) * u)
    if act == "bf16":
        hq = [bf16_nearest(v) for v in h]
        hh = [float(bf16_value(b & 0x7FFF)) * (-1.0 if b & 0x8000 else 1.0) for b in hq]
        return [_dot(r, hh) for r in rows2], hq, None
    hh, hq, hs = _quantize_dequant(h)
    return [_dot(r, hh) for r in rows2], hq, hs


def brute_ref(x_bits, topk_ids, topk_weights, w13, w13_s, w2, w2_s, shared=None, act="fp8"):
    """Same contract as ``moe.ffn_ref`` (all tokens) for tiny numpy inputs.
    Returns y (float64 [T, H]) and h codes/scales per (token, pick). act="bf16":
    x used as its bf16 values, h rounded to bf16 (h_q uint16 bit patterns)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    K = topk_ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    y = np.zeros((T, H))
    hq_all = np.zeros((T, K, I), dtype=np.uint16 if act == "bf16" else np.uint8)
    hs_all = np.zeros((T, K, I // 128), dtype=np.uint8)
    cache = {}
    for t in range(T):
        if act == "bf16":
            xh = [float(bf16_value(int(b) & 0x7FFF)) * (-1.0 if int(b) & 0x8000 else 1.0) for b in x_bits[t]]
        else:
            xh, xq, xs = _quantize_dequant([bf16_value(int(b)) for b in x_bits[t]])
        terms = [[] for _ in range(H)]
        for j in range(K):
            e = int(topk_ids[t, j])
            if not (0 <= e < E):
                continue
            if e not in cache:
                cache[e] = (_floats(mxfp4_row(w13[e, n], w13_s[e, n]) for n in range(2 * I)),
                            _floats(mxfp4_row(w2[e, n], w2_s[e, n]) for n in range(H)))
            o, hq, hs = _expert(xh, cache[e][0], cache[e][1], I, act)
            hq_all[t, j] = hq
            if hs is not None:
                hs_all[t, j] = hs
            wt = float(topk_weights[t, j])
            for n in range(H):
                terms[n].append(wt * o[n])
        if shared is not None:
            Is = shared["w2s"].shape[1]
            if "rows" not in cache:
                cache["rows"] = (
                    _floats(fp8_block_row(shared["w13s"][n], shared["w13s_s"], n) for n in range(2 * Is)),
                    _floats(fp8_block_row(shared["w2s"][n], shared["w2s_s"], n) for n in range(H)))
            o, _, _ = _expert(xh, cache["rows"][0], cache["rows"][1], Is)
            for n in range(H):
                terms[n].append(o[n])
        for n in range(H):
            y[t, n] = math.fsum(terms[n])
    return {"y": y, "h_q": hq_all, "h_s": hs_all}


def brute_ref_nvfp4(x_bits, topk_ids, topk_weights, w13, w13_s, w13_gs, w2, w2_s, w2_gs):
    """Same contract as ``moe.ffn_ref_nvfp4`` (all tokens), written from the
    element definitions: every weight is E2M1 x E4M3 x tensor scale as an exact
    fraction (its float has at most 30 significant bits, so every product with a
    bf16 activation is exact in float64), dots by fsum, bf16 rounding by bisection."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    K = topk_ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    y = np.zeros((T, H))
    hq_all = np.zeros((T, K, I), dtype=np.uint16)
    cache = {}
    for t in range(T):
        xh = [float(bf16_value(int(b) & 0x7FFF)) * (-1.0 if int(b) & 0x8000 else 1.0) for b in x_bits[t]]
        terms = [[] for _ in range(H)]
        for j in range(K):
            e = int(topk_ids[t, j])
            if not (0 <= e < E):
                continue
            if e not in cache:
                cache[e] = (_floats(nvfp4_row(w13[e, n], w13_s[e, n], w13_gs[e]) for n in range(2 * I)),
                            _floats(nvfp4_row(w2[e, n], w2_s[e, n], w2_gs[e]) for n in range(H)))
            o, hq, _ = _expert(xh, cache[e][0], cache[e][1], I, "bf16")
            hq_all[t, j] = hq
            wt = float(topk_weights[t, j])
            for n in range(H):
                terms[n].append(wt * o[n])
        for n in range(H):
            y[t, n] = math.fsum(terms[n])
    return {"y": y, "h_q": hq_all}
