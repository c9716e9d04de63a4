"""Parity metrics between a GPU result and the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Final output y (bf16): relative error of the whole tensor against the float64
  oracle, max_rel = max|y - r| / max|r| and mean_rel = sum|y - r| / sum|r|, and
  the largest per-row max_rel. Elementwise ratios are not used: they blow up
  where r is near zero. Rounding y to bf16 alone already gives mean_rel near
  1.4e-3 on these workloads.
* SwiGLU-output FP8 codes. The bar: at most 1 grid step of difference on at
  most 0.1% of the elements. ``h_code_mismatch`` sorts every element into
    equal       -- same decoded value (+0 and -0 are equal);
    one_step    -- same block scale, grid positions one apart;
    scale_flip  -- a block scale that differs where the oracle's block amax sits
                   within 2^-16 (relative) of a scale boundary 1.75 * 2^p, and
                   values at most one grid step of the coarser scale apart;
    beyond      -- any other difference. With an ``envelope`` (the exact SwiGLU
                   value and a rigorous bound on the GPU's deviation from it,
                   oracle/envelope.py) a beyond element is ``in_envelope`` when
                   its code rounds from a value inside that bound under the GPU's
                   block scale (and, where that scale differs, the block's exact
                   amax lies within the block's largest bound of a boundary);
                   otherwise, and always without an envelope, it is ``bad``.
  Tests require bad == 0, frac_differ <= 0.1% and beyond at most a small cap.
* SwiGLU outputs of the bf16-activation variant (bf16 bit patterns):
  ``h_bf16_mismatch`` sorts them into equal / one_ulp (adjacent bf16 values,
  across zero too) / beyond; with an envelope every differing element (one ulp
  or more) is checked to be the bf16 rounding (nearest, ties to even, which is
  monotone) of some value inside the bound, so that each difference is explained
  by the GPU's arithmetic and none by a wrong result.
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
    row_rel = d.max(axis=-1) / np.maximum(np.abs(r).max(axis=-1), 1e-300) if d.size else np.zeros(1)
    return {
        "max_rel": float(d.max() / max(np.abs(r).max(), 1e-300)) if d.size else 0.0,
        "mean_rel": float(d.sum() / max(np.abs(r).sum(), 1e-300)) if d.size else 0.0,
        "row_max_rel": float(row_rel.max()) if d.size else 0.0,
        "frac_equal_bf16": float(eq.mean()) if eq.size else 1.0,
        "finite": bool(np.isfinite(y).all()),
    }


def _signed_index(codes: np.ndarray) -> np.ndarray:
    """E4M3 code -> signed position on the grid (+-0 -> 0); adjacent grid points
    differ by 1, across zero too."""
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def _boundary_distance(amax: np.ndarray) -> np.ndarray:
    """|amax - 1.75 * 2^p| for the boundary in amax's binade (amax = m * 2^p)."""
    _, ex = np.frexp(amax)               # amax = 2m * 2^(ex-1)
    return np.abs(amax - 1.75 * np.ldexp(1.0, ex - 1))


def h_code_mismatch(hq, hs, hq_ref, hs_ref, amax_ref, block: int = 128, envelope=None) -> dict:
    """Compare SwiGLU-output codes element by element (categories in the module
    docstring).

    hq, hq_ref uint8 [R, C]; hs, hs_ref uint8 [R, C/block]; amax_ref float64
    [R, C/block] (the oracle's block amax). ``envelope``: optional callable
    (rows, cols) -> (h_exact, h_err), float64 arrays for the listed elements.
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
    va = E4M3_VALUES[a] * np.ldexp(1.0, hs - 127)[..., None]
    vb = E4M3_VALUES[b] * np.ldexp(1.0, hs_ref - 127)[..., None]
    equal = va == vb
    same = (hs == hs_ref)[..., None]
    dist = np.abs(_signed_index(a) - _signed_index(b))
    one_step = ~equal & same & (dist == 1)

    near = _boundary_distance(amax) <= amax * 2.0 ** -16
    coarse = np.ldexp(1.0, np.maximum(hs, hs_ref) - 127)[..., None]
    mag = np.maximum(np.abs(va), np.abs(vb)) / coarse
    _, mex = np.frexp(np.maximum(mag, 2.0 ** -6))
    step = np.ldexp(1.0, mex - 1 - 3) * coarse
    scale_flip = ~equal & ~same & near[..., None] & (np.abs(va - vb) <= step)

    beyond = ~equal & ~one_step & ~scale_flip
    in_env = np.zeros_like(beyond)
    if envelope is not None and beyond.any():
        # every element of a block whose scale differs is needed for its amax bound
        blk_rows, blk_ids = np.nonzero(beyond.any(axis=-1))
        cols = (blk_ids[:, None] * block + np.arange(block)[None, :]).ravel()
        rows = np.repeat(blk_rows, block)
        h, err = envelope(rows, cols)
        h = np.asarray(h, np.float64).reshape(-1, block)
        err = np.asarray(err, np.float64).reshape(-1, block)
        sg = hs[blk_rows, blk_ids]
        lo = e4m3_encode(np.ldexp(h - err, -(sg - 127)[:, None]))
        hi = e4m3_encode(np.ldexp(h + err, -(sg - 127)[:, None]))
        ia = _signed_index(a[blk_rows, blk_ids])
        ok = (ia >= _signed_index(lo)) & (ia <= _signed_index(hi))
        exact_amax = np.abs(h).max(axis=-1)
        scale_ok = (sg == hs_ref[blk_rows, blk_ids]) | (_boundary_distance(exact_amax) <= err.max(axis=-1))
        in_env[blk_rows, blk_ids] = ok & scale_ok[:, None]
    in_env &= beyond
    bad = beyond & ~in_env

    n = int(a.size)
    idx = np.argwhere(bad)[:5]
    examples = [(int(a[i, j, k]), int(b[i, j, k]), float(va[i, j, k]), float(vb[i, j, k]), float(amax[i, j]))
                for i, j, k in idx]
    differ = int((~equal).sum())
    return {"elements": n, "differ": differ, "frac_differ": differ / max(n, 1),
            "one_step": int(one_step.sum()), "scale_flip": int(scale_flip.sum()),
            "beyond": int(beyond.sum()), "in_envelope": int(in_env.sum()), "bad": int(bad.sum()),
            "scale_diff_blocks": int((~same[..., 0]).sum()),
            "max_code_dist_same_scale": int(np.where(same, dist, 0).max()) if n else 0,
            "bad_examples": examples}


def _bf16_index(bits: np.ndarray) -> np.ndarray:
    """bf16 pattern -> signed position on the ordered bf16 line (+-0 -> 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def h_bf16_mismatch(hb, hb_ref, envelope=None) -> dict:
    """hb, hb_ref: bf16 bit patterns of the same shape [R, C] (GPU, oracle).
    envelope(rows, cols) -> (h_exact, h_err) float64 arrays: the exact SwiGLU
    value of each listed element and a bound on the GPU's deviation from it
    before its rounding to bf16."""
    a = np.asarray(hb, dtype=np.uint16)
    r = np.asarray(hb_ref, dtype=np.uint16)
    ia, ir = _bf16_index(a), _bf16_index(r)
    dist = np.abs(ia - ir)
    differ = dist != 0
    rows, cols = np.nonzero(differ)
    out = {"elements": int(a.size), "differ": int(differ.sum()),
           "frac_differ": float(differ.mean()) if a.size else 0.0,
           "one_ulp": int((dist == 1).sum()), "beyond": int((dist > 1).sum()),
           "max_ulp": int(dist.max()) if a.size else 0, "in_envelope": 0, "bad": 0, "bad_examples": []}
    if rows.size == 0:
        return out
    if envelope is None:
        out["bad"] = out["beyond"]
        bi = np.nonzero(dist[rows, cols] > 1)[0][:5]
        out["bad_examples"] = [(int(rows[i]), int(cols[i]), int(a[rows[i], cols[i]]), int(r[rows[i], cols[i]]))
                               for i in bi]
        return out
    h, e = envelope(rows, cols)
    lo = _bf16_index(f64_to_bf16_rne(h - e))
    hi = _bf16_index(f64_to_bf16_rne(h + e))
    g = ia[rows, cols]
    ok = (g >= lo) & (g <= hi)
    out["in_envelope"] = int(ok.sum())
    out["bad"] = int((~ok).sum())
    bi = np.nonzero(~ok)[0][:5]
    out["bad_examples"] = [(int(rows[i]), int(cols[i]), int(a[rows[i], cols[i]]), int(r[rows[i], cols[i]]),
                            float(h[i]), float(e[i])) for i in bi]
    return out
