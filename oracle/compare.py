"""Parity metrics between a GPU result and the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Final output y (bf16): relative error of the whole tensor against the float64
  oracle, max_rel = max|y - r| / max|r| and mean_rel = sum|y - r| / sum|r|.
  Elementwise ratios are not used: they blow up where r is near zero. Rounding
  y to bf16 alone already gives mean_rel near 1.4e-3 on these workloads.
* SwiGLU-output FP8 codes: the GPU evaluates the W13 GEMM in fp32 and silu with
  its own exp, so a code may land one grid step away from the oracle's, and a
  block whose amax sits right at a scale boundary (1.75 * 2^p) may take the
  neighbouring scale. ``h_code_mismatch`` counts the elements that differ by
  more than that.
"""

from __future__ import annotations

import numpy as np

from .formats import E4M3_VALUES, bf16_to_f64, e4m3_encode, f64_to_bf16_rne


def y_metrics(y_bits: np.ndarray, y_ref: np.ndarray) -> dict:
    """y_bits: bf16 bit patterns [n, H]; y_ref float64 [n, H]."""
    y = bf16_to_f64(y_bits)
    r = np.asarray(y_ref, dtype=np.float64)
    d = np.abs(y - r)
    eq = (np.asarray(y_bits, dtype=np.uint16) == f64_to_bf16_rne(r))
    return {
        "max_rel": float(d.max() / max(np.abs(r).max(), 1e-300)) if d.size else 0.0,
        "mean_rel": float(d.sum() / max(np.abs(r).sum(), 1e-300)) if d.size else 0.0,
        "frac_equal_bf16": float(eq.mean()) if eq.size else 1.0,
        "finite": bool(np.isfinite(y).all()),
    }


def _signed_index(codes: np.ndarray) -> np.ndarray:
    """E4M3 code -> signed position on the grid (+-0 -> 0); adjacent grid points
    differ by 1, across zero too."""
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def h_code_mismatch(hq, hs, hq_ref, hs_ref, amax_ref, block: int = 128, h_ref=None, h_err=None) -> dict:
    """Compare SwiGLU-output codes element by element.

    hq, hq_ref uint8 [R, C]; hs, hs_ref uint8 [R, C/block]; amax_ref float64
    [R, C/block] (the oracle's block amax). Each element is
      equal  -- same decoded value (+0 and -0 are equal);
      close  -- the values are neighbours:
                * same scale and grid positions one apart; or
                * same scale, both values at most 2^-5 * scale in magnitude (the
                  E4M3 grid is uniform with step 2^-9 * scale from 0 up to and
                  including 2^-5 * scale, finer there than the rounding inside a
                  hardware MX dot product) and at most 2^-6 * scale apart; or
                * a scale that differs in a block whose oracle amax is within
                  2^-16 (relative) of a scale boundary 1.75 * 2^p, and values at
                  most one grid step of the coarser scale apart;
                * with an envelope (h_ref, the exact values, and h_err >= 0): same
                  scale and a code between the codes of h_ref - h_err and
                  h_ref + h_err (the value rounds from somewhere in the envelope);
                  the scale-boundary window widens to the block's largest h_err;
      bad    -- anything else (a scale that differs away from a boundary makes
                every element of its block bad).
    The bar: no bad element, and at most 0.1% of elements close-but-unequal.
    """
    hq = np.asarray(hq).reshape(-1, np.asarray(hq).shape[-1])
    hq_ref = np.asarray(hq_ref).reshape(hq.shape)
    R, C = hq.shape
    nb = C // block
    hs = np.asarray(hs).reshape(R, nb).astype(np.int64)
    hs_ref = np.asarray(hs_ref).reshape(R, nb).astype(np.int64)
    amax = np.asarray(amax_ref, dtype=np.float64).reshape(R, nb)

    a = hq.reshape(R, nb, block)
    b = hq_ref.reshape(R, nb, block)
    scale_a = np.ldexp(1.0, hs - 127)[..., None]
    scale_b = np.ldexp(1.0, hs_ref - 127)[..., None]
    va = E4M3_VALUES[a] * scale_a
    vb = E4M3_VALUES[b] * scale_b
    equal = va == vb
    same = (hs == hs_ref)[..., None]
    dist = np.abs(_signed_index(a) - _signed_index(b))
    fixed_step = (np.abs(E4M3_VALUES[a]) <= 2.0 ** -5) & (np.abs(E4M3_VALUES[b]) <= 2.0 ** -5) & \
        (np.abs(va - vb) <= 2.0 ** -6 * scale_b)

    in_env = np.zeros_like(equal)
    window = amax * 2.0 ** -16
    if h_ref is not None:
        hr = np.asarray(h_ref, dtype=np.float64).reshape(R, nb, block)
        he = np.asarray(h_err, dtype=np.float64).reshape(R, nb, block)
        lo = e4m3_encode(np.ldexp(hr - he, -(hs_ref - 127)[..., None]))
        hi = e4m3_encode(np.ldexp(hr + he, -(hs_ref - 127)[..., None]))
        ia, ilo, ihi = _signed_index(a), _signed_index(lo), _signed_index(hi)
        in_env = (ia >= np.minimum(ilo, ihi)) & (ia <= np.maximum(ilo, ihi))
        window = np.maximum(window, he.max(axis=-1))
    _, ex = np.frexp(amax)               # amax = 2m * 2^(ex-1)
    boundary = 1.75 * np.ldexp(1.0, ex - 1)
    near = np.abs(amax - boundary) <= window
    coarse = np.ldexp(1.0, np.maximum(hs, hs_ref) - 127)[..., None]
    mag = np.maximum(np.abs(va), np.abs(vb)) / coarse
    _, mex = np.frexp(np.maximum(mag, 2.0 ** -6))
    step = np.ldexp(1.0, mex - 1 - 3) * coarse
    close_diff = near[..., None] & (np.abs(va - vb) <= step)

    close = ~equal & np.where(same, (dist <= 1) | fixed_step | in_env, close_diff)
    bad = ~equal & ~close
    n = int(a.size)
    idx = np.argwhere(bad)[:5]
    examples = [(int(a[i, j, k]), int(b[i, j, k]), float(va[i, j, k]), float(vb[i, j, k]), float(amax[i, j]))
                for i, j, k in idx]
    return {"elements": n, "bad_examples": examples, "differ": int((~equal).sum()), "bad": int(bad.sum()),
            "frac_differ": float((~equal).sum()) / max(n, 1),
            "scale_diff_blocks": int((~same[..., 0]).sum()),
            "max_code_dist_same_scale": int(np.where(same, dist, 0).max()) if n else 0}
