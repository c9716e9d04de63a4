"""Pins for oracle/compare.py: planted differences are classified as documented."""

import numpy as np

from oracle.compare import h_code_mismatch, y_metrics
from oracle.formats import e4m3_encode, f64_to_bf16_rne, quantize_blocks


def _blocks(seed=0, R=8, C=256):
    v = np.random.default_rng(seed).standard_normal((R, C))
    return quantize_blocks(v)


def test_identical_codes():
    q, s, a = _blocks()
    m = h_code_mismatch(q, s, q, s, a)
    assert m["differ"] == 0 and m["bad"] == 0


def test_one_step_is_close_two_steps_is_bad():
    q, s, a = _blocks()
    g = q.copy()
    big = np.argwhere((q & 0x7F) > 0x40)[:2]
    g[tuple(big[0])] += 1                       # one grid step
    g[tuple(big[1])] += 2                       # two grid steps, normal range
    m = h_code_mismatch(g, s, q, s, a)
    assert m["differ"] == 2 and m["bad"] == 1


def test_fixed_step_region():
    q, s, a = _blocks()
    g = q.copy()
    g[0, 0], q2 = 0x0A, q.copy()
    q2[0, 0] = 0x08                             # 1.25 * 2^-6 vs 2^-6: two 2^-9 steps apart
    m = h_code_mismatch(g, s, q2, s, a)
    assert m["bad"] == 0 and m["differ"] == 1
    g[0, 0] = 0x12                              # 2^-5 * 1.25: outside the fixed-step region
    assert h_code_mismatch(g, s, q2, s, a)["bad"] == 1
    # the region's top end, 2^-5 (code 0x10), is still on the uniform 2^-9 grid:
    # 0x0E = 1.75 * 2^-6 lies two steps below it
    g[0, 0], q2[0, 0] = 0x8E, 0x90
    m = h_code_mismatch(g, s, q2, s, a)
    assert m["bad"] == 0 and m["differ"] == 1
    g[0, 0], q2[0, 0] = 0x90, 0x92              # 2^-5 vs 1.25 * 2^-5: step 2^-8 above the region
    assert h_code_mismatch(g, s, q2, s, a)["bad"] == 1


def test_sign_of_zero_is_equal_and_scale_flip_away_from_boundary_is_bad():
    q, s, a = _blocks()
    g = q.copy()
    z = np.argwhere(q == 0)
    if z.size:
        g[tuple(z[0])] = 0x80
    assert h_code_mismatch(g, s, q, s, a)["differ"] == 0
    s2 = s.copy()
    s2[0, 0] += 1
    m = h_code_mismatch(q, s2, q, s, a)
    assert m["bad"] >= 100


def test_y_metrics():
    r = np.random.default_rng(1).standard_normal((16, 64))
    m = y_metrics(f64_to_bf16_rne(r), r)
    assert m["frac_equal_bf16"] == 1.0 and m["mean_rel"] < 4e-3 and m["max_rel"] < 4e-3
    m2 = y_metrics(f64_to_bf16_rne(2 * r), r)
    assert abs(m2["mean_rel"] - 1.0) < 1e-2


def test_envelope_accepts_codes_reachable_from_the_envelope_only():
    """A code two grid steps from the oracle's is accepted only when the
    envelope [h - err, h + err] around the exact value reaches it (scale 2^-8,
    binade [2^-5, 2^-4) of the scaled grid: step 2^-8 * 2^-8)."""
    R, C = 1, 128
    scale_code = np.array([[119]], dtype=np.uint8)            # 2^-8
    amax = np.array([[1.19]])
    h = np.zeros((R, C))
    h[0, 0] = -1.75 * 2.0 ** -5 * 2.0 ** -8                    # exactly code 0x96 after scaling
    ref = e4m3_encode(np.ldexp(h, 8))
    assert ref[0, 0] == 0x96
    gpu = ref.copy()
    gpu[0, 0] = 0x98                                           # -2^-4 * 2^-8: two steps away
    err_wide = np.full((R, C), 4e-5)
    m = h_code_mismatch(gpu, scale_code, ref, scale_code, amax, h_ref=h, h_err=err_wide)
    assert m["bad"] == 0 and m["differ"] == 1
    m = h_code_mismatch(gpu, scale_code, ref, scale_code, amax, h_ref=h, h_err=np.full((R, C), 1e-6))
    assert m["bad"] == 1
    m = h_code_mismatch(gpu, scale_code, ref, scale_code, amax)  # no envelope: the default rules
    assert m["bad"] == 1
