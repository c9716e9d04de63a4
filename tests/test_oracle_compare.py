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


def test_two_steps_near_zero_are_beyond_without_an_envelope():
    """The former fixed-step region is gone: near zero, two grid steps are two
    steps (counted beyond, bad without an envelope)."""
    q, s, a = _blocks()
    g, q2 = q.copy(), q.copy()
    g[0, 0], q2[0, 0] = 0x0A, 0x08             # 1.25 * 2^-6 vs 2^-6: two 2^-9 steps
    m = h_code_mismatch(g, s, q2, s, a)
    assert m["beyond"] == 1 and m["bad"] == 1 and m["one_step"] == 0


def test_categories_are_counted():
    q, s, a = _blocks(R=4, C=256)
    g = q.copy()
    big = np.argwhere((q & 0x7F) > 0x40)
    g[tuple(big[0])] += 1
    g[tuple(big[1])] += 1
    g[tuple(big[2])] += 3
    m = h_code_mismatch(g, s, q, s, a)
    assert (m["differ"], m["one_step"], m["beyond"], m["bad"]) == (3, 2, 1, 1)
    assert m["max_code_dist_same_scale"] == 3 and abs(m["frac_differ"] - 3 / q.size) < 1e-15


def _envelope_case():
    """One block, scale 2^-8 (code 119); the exact value sits exactly on code
    0x96 = -1.75 * 2^-5 of the scaled grid (step 2^-8 there)."""
    R, C = 1, 128
    scale_code = np.array([[119]], dtype=np.uint8)
    amax = np.array([[1.19]])
    h = np.zeros((R, C))
    h[0, 0] = -1.75 * 2.0 ** -5 * 2.0 ** -8
    h[0, 1] = 1.19                              # the block's amax element (code unchanged)
    ref = e4m3_encode(np.ldexp(h, 8))
    assert ref[0, 0] == 0x96
    gpu = ref.copy()
    gpu[0, 0] = 0x98                            # -2^-4 * 2^-8: two steps away
    return gpu, scale_code, ref, amax, h


def test_envelope_accepts_codes_reachable_from_the_envelope_only():
    gpu, sc, ref, amax, h = _envelope_case()
    calls = []

    def env_of(err):
        def f(rows, cols):
            calls.append((rows.copy(), cols.copy()))
            return h[rows, cols], np.full(rows.size, err)
        return f

    m = h_code_mismatch(gpu, sc, ref, sc, amax, envelope=env_of(4e-5))
    assert (m["beyond"], m["in_envelope"], m["bad"]) == (1, 1, 0)
    # the envelope is asked for the whole block of the beyond element only
    assert np.array_equal(calls[0][0], np.zeros(128)) and np.array_equal(calls[0][1], np.arange(128))
    m = h_code_mismatch(gpu, sc, ref, sc, amax, envelope=env_of(1e-6))
    assert (m["in_envelope"], m["bad"]) == (0, 1)
    assert h_code_mismatch(gpu, sc, ref, sc, amax)["bad"] == 1


def test_envelope_scale_change_needs_amax_near_a_boundary():
    """A GPU block scale one above the oracle's: accepted through the envelope only
    when the block's exact amax lies within the block's largest bound of a scale
    boundary and every code rounds from inside the envelope under the GPU scale."""
    R, C = 1, 128
    h = np.random.default_rng(4).uniform(-1, 1, (R, C))
    h[0, 7] = 1.75 * (1 - 2.0 ** -12)           # amax just below the boundary 1.75
    qr, sr, ar = quantize_blocks(h)
    qg, sg, _ = quantize_blocks(h * (1 + 2.0 ** -11))   # the GPU's values crossed it
    assert sg[0, 0] == sr[0, 0] + 1

    def env_of(err):
        return lambda rows, cols: (h[rows, cols], np.full(rows.size, err))

    # 2^-16-relative window of the plain rule does not cover this amax distance
    assert h_code_mismatch(qg, sg, qr, sr, ar)["bad"] > 0
    m = h_code_mismatch(qg, sg, qr, sr, ar, envelope=env_of(2.0 ** -10))
    assert m["bad"] == 0 and m["in_envelope"] == m["beyond"] > 0
    m = h_code_mismatch(qg, sg, qr, sr, ar, envelope=env_of(2.0 ** -16))
    assert m["bad"] > 0


# ----------------------------------------------------------------------------- bf16 SwiGLU outputs

from oracle.compare import h_bf16_mismatch  # noqa: E402
from oracle.formats import bf16_to_f64 as _b2f, f64_to_bf16_rne as _f2b  # noqa: E402


def _bf(vals):
    return _f2b(np.asarray(vals, np.float64)).reshape(1, -1)


def test_bf16_categories_without_envelope():
    ref = _bf([1.0, -2.0, 0.0, 3.0, 1e-3])
    gpu = ref.copy()
    gpu[0, 0] += 1                         # one ulp up
    gpu[0, 2] = 0x8001                     # -0 -> smallest negative subnormal: one ulp across zero
    gpu[0, 3] += 2                         # two ulps: beyond, bad without an envelope
    m = h_bf16_mismatch(gpu, ref)
    assert (m["differ"], m["one_ulp"], m["beyond"], m["bad"], m["max_ulp"]) == (3, 2, 1, 1, 2)
    assert m["bad_examples"][0][:2] == (0, 3)
    assert h_bf16_mismatch(ref, ref)["differ"] == 0
    assert h_bf16_mismatch(_bf([0.0]), np.array([[0x8000]], np.uint16))["differ"] == 0


def test_bf16_envelope_explains_or_rejects_each_difference():
    h = np.array([1.0 + 2.0 ** -8 - 2.0 ** -20, 5.0, 5.0])    # just below a rounding boundary; mid-step
    ref = _f2b(h).reshape(1, -1)
    gpu = ref.copy()
    gpu[0, 0] += 1                         # reachable: h + 2^-19 rounds up
    gpu[0, 1] += 1                         # one ulp from a value far from any boundary: wrong
    gpu[0, 2] += 3                         # three ulps, reachable only with a wide bound

    def env_fn(err):
        return lambda rows, cols: (h[cols], np.asarray(err)[cols])

    m = h_bf16_mismatch(gpu, ref, envelope=env_fn([2.0 ** -19, 2.0 ** -19, 2.0 ** -19]))
    assert (m["in_envelope"], m["bad"]) == (1, 2)
    m = h_bf16_mismatch(gpu, ref, envelope=env_fn([2.0 ** -19, 2.0 ** -19, 0.1]))
    assert (m["in_envelope"], m["bad"]) == (2, 1)
    assert m["bad_examples"][0][1] == 1
    assert _b2f(gpu)[0, 2] <= 5.1
