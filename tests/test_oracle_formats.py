"""Pins for oracle/formats.py: decode tables, E4M3 rounding, the block-scale rule.

Pinned against things other than the oracle itself:
  * closed-form properties of the OCP formats (hand-written fixture in
    tests/golden/ocp_formats.json),
  * torch's own float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions (an
    independent library implementation of the same OCP formats),
  * the brute-force nearest-code search and exponent search in oracle/brute.py.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import brute
from oracle.formats import (E2M1_VALUES, E4M3_VALUES, E8M0_VALUES, bf16_to_f64, dequantize_blocks,
                            e4m3_encode, f64_to_bf16_rne, quantize_blocks, scale_exponent)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ocp_formats.json")))

ALL_BF16 = np.arange(65536, dtype=np.uint16)
ALL_BF16_VALUES = bf16_to_f64(ALL_BF16)
FINITE = np.isfinite(ALL_BF16_VALUES)


def test_e2m1_table_closed_form():
    assert sorted(set(np.abs(E2M1_VALUES).tolist())) == GOLD["e2m1_magnitudes"]
    for c in range(16):
        assert E2M1_VALUES[c] == float(brute.e2m1(c))
        assert np.signbit(E2M1_VALUES[c]) == bool(c & 8)
    assert E2M1_VALUES[8] == 0.0 and np.signbit(E2M1_VALUES[8])        # code 8 is -0


def test_e4m3_table_closed_form_and_library():
    v = E4M3_VALUES
    assert v[0x7E] == GOLD["e4m3_max"]
    assert v[0x01] == 2.0 ** GOLD["e4m3_min_subnormal_exp"]
    assert v[0x08] == 2.0 ** GOLD["e4m3_min_normal_exp"]
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[1:0x7F]
    assert pos.size == GOLD["e4m3_positive_finite_nonzero"] and np.all(np.diff(pos) > 0)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = ~np.isnan(lib)
    assert np.array_equal(np.isnan(v), ~fin)
    assert np.array_equal(v[fin], lib[fin])
    assert np.array_equal(np.signbit(v[fin]), np.signbit(lib[fin]))
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert v[c] == float(brute.e4m3(c))


def test_e8m0_table_library():
    lib = torch.arange(255, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(E8M0_VALUES[:255], lib)
    assert E8M0_VALUES[127] == 1.0 and np.isnan(E8M0_VALUES[255])


@pytest.mark.parametrize("e", list(range(-20, 21)))
def test_e4m3_encode_exhaustive_vs_torch(e):
    """Every finite bf16 value divided by 2^e, against torch's RNE cast (torch
    does not saturate, so compare where |v| < 464, the rounding midpoint above 448)."""
    s = np.ldexp(ALL_BF16_VALUES[FINITE], -e)
    m = np.abs(s) < 464
    ref = torch.from_numpy(s[m]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(s[m]), ref)


def test_e4m3_encode_vs_bruteforce_nearest():
    rng = np.random.default_rng(7)
    grid = E4M3_VALUES[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2                     # exact ties
    vals = np.concatenate([mids, -mids, rng.uniform(-460, 460, 300),
                           rng.uniform(-2.0 ** -5, 2.0 ** -5, 200), [0.0, -0.0, 500.0, -1e9, 2.0 ** -11]])
    got = e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert g == brute.e4m3_nearest(Fraction(float(v)), bool(np.signbit(v))), v


def test_e4m3_encode_saturates_and_keeps_sign_of_zero():
    assert e4m3_encode(np.array([449.0, 1e30, -1e30]))[0] == 0x7E
    assert e4m3_encode(np.array([-1e30]))[0] == 0xFE
    assert e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert e4m3_encode(np.array([-2.0 ** -11]))[0] == 0x80


def test_scale_exponent_exhaustive_vs_search():
    """All positive finite bf16 amax values vs an exponent search (vectorised
    brute force: the first e in [-127, 127] with amax <= 448 * 2^e)."""
    a = ALL_BF16_VALUES[FINITE & (ALL_BF16_VALUES >= 0)]
    es = np.arange(-127, 128)
    fits = a[:, None] <= 448.0 * np.ldexp(1.0, es)[None, :]
    first = np.where(fits.any(1), es[np.argmax(fits, axis=1)], 127)
    assert np.array_equal(scale_exponent(a), first)
    # spot-check the brute-force module's exact-fraction search too
    for v in a[::997]:
        assert scale_exponent(np.array([v]))[0] == brute.block_scale(Fraction(float(v)))


def test_quantize_blocks_never_saturates_and_roundtrips():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-30, 30, (64, 1)))
    codes, sc, amax = quantize_blocks(x)
    mag = np.abs(E4M3_VALUES[codes]).reshape(64, 4, 128).max(-1)
    # amax / 2^e lies in (224, 448]; rounding can bring the largest code down to 224
    assert np.all(mag >= 224) and np.all(mag <= 448)
    # values already on the grid survive a round trip (a block whose largest code
    # rounded down to 224 re-quantizes with half the scale, same values)
    back = dequantize_blocks(codes, sc)
    c2, s2, _ = quantize_blocks(back)
    assert np.array_equal(dequantize_blocks(c2, s2), back)
    keep = (mag > 224)
    assert np.array_equal(s2[keep], sc[keep]) and np.all(s2[~keep] == sc[~keep] - 1)
    # the zero block takes the smallest scale and zero codes
    z, zs, _ = quantize_blocks(np.zeros((1, 128)))
    assert zs[0, 0] == 0 and not z.any()


def test_bf16_rounding_vs_torch():
    """Against torch's float32 -> bfloat16 cast (one rounding; torch's float64 ->
    bfloat16 goes through float32 and can round twice, so it is not the pin)."""
    x = (torch.randn(200000) * torch.exp(torch.empty(200000).uniform_(-40, 40))).float()
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_rne(x.double().numpy()), ref)
    assert np.array_equal(bf16_to_f64(ref), x.to(torch.bfloat16).double().numpy())
