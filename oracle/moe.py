"""Oracle for the routed MoE FFN (plain CPU, float64, exact dequantization).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed (per token t, with e = topk_ids[t, j]):

    y_t = sum_j w[t, j] * W2[e] . Q( silu(W1[e] . Q(x_t)) * (W3[e] . Q(x_t)) )
          (+ the shared expert's output, weight 1)

* Q(.) quantizes a vector to E4M3 with one power-of-two scale per 128
  consecutive elements and dequantizes it again (``formats.quantize_blocks``).
  For x this is the online FP8 activation quantization ("Pushing the Limits of
  Serving DeepSeek-V4-Pro", §2.2); for the SwiGLU output it is the quantization
  fused with SwiGLU that hands W2 its FP8 data and scales (same blog, §4.3). The
  routing weight is applied after W2, in the top-k reduction (same blog, §3.2),
  so the SwiGLU output is quantized unweighted.
* W1 = W13 rows [0, I) (gate), W3 = W13 rows [I, 2I) (up), W2 the down
  projection; all MXFP4, dequantized exactly (E2M1 value * 2^(scale-127)).
* silu(g) = g / (1 + exp(-g)), evaluated in float64, no clamp.

MXFP4A16 variant (``act="bf16"``; MXFP4 weights with 16-bit activations, the
variant the "Pushing the Limits of Serving DeepSeek-V4-Pro" blog compares against
in Appendix D.2): x is used as its exact bf16 values, not quantized, and W2 takes
B(silu(g) * u), the SwiGLU output rounded once to bf16 (nearest, ties to even).
Reading: the page names the variant only; 16-bit activations mean the operands of
both GEMMs are bf16, and the SwiGLU output is rounded once where it becomes W2's
operand, as in the FP8 form where that is the FP8 quantization.

NVFP4 weights (``ffn_ref_nvfp4``; "Optimization progress report", Optimization
05: NVFP4 expert weights consumed as stored). The page names the format only; it
is NVIDIA's published NVFP4: E2M1 codes, one E4M3 scale per 16 consecutive
elements and one fp32 scale per tensor (here per expert and projection),
w = E2M1 * E4M3 * tensor scale. Reading: activations bf16 as in the variant
above (the page names no activation format). The tensor scale is constant over
each contraction, so it multiplies the exact dot product once; that keeps the
GEMMs exact (E2M1 * E4M3 has at most 6 significant bits).

Exactness: a product of an E4M3 value (4 significant bits) and an E2M1 value
(2 significant bits) times power-of-two scales has at most 6 significant bits,
and a dot product over 7168 such terms spans far fewer than float64's 53 bits
for realistic scales, so the float64 GEMMs below are exact whatever order the
BLAS library sums in (tests/test_oracle_ffn.py checks this against math.fsum).
The same holds for bf16 activations (8 significant bits; products of 10) at
realistic value spreads, checked the same way.
The oracle therefore fixes the GEMM results exactly; only exp and the final
combine carry float64 rounding.
"""

from __future__ import annotations

import numpy as np
import torch

from .formats import (E2M1_VALUES, E4M3_VALUES, E8M0_VALUES, bf16_to_f64,
                      dequantize_blocks, f64_to_bf16_rne, quantize_blocks)

# ----------------------------------------------------------------------------- plan


def plan_ref(topk_ids, E: int) -> dict:
    """Route plan: pack the (token, pick) pairs by expert ahead of the expert GEMMs
    without changing the token-to-expert mapping ("Optimization progress report",
    Optimization 14).

    Pair p = t*K + j. Reading (the pages give no order): pairs are ordered by
    expert and, within an expert, by p (a stable sort). Ids outside [0, E) are
    dropped and counted. Returns
      expert_offsets [E+1] int32  -- exclusive scan of per-expert counts
      sorted_pairs   [P]   int32  -- pair ids in plan order, -1 past the valid ones
      pair_rows      [P]   int32  -- position of pair p in sorted_pairs, -1 if dropped
      dropped        int
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    P = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(np.where(valid, ids, E), kind="stable")
    n = int(valid.sum())
    sorted_pairs = np.full(P, -1, dtype=np.int32)
    sorted_pairs[:n] = order[:n]
    pair_rows = np.full(P, -1, dtype=np.int32)
    pair_rows[order[:n]] = np.arange(n, dtype=np.int32)
    return {"expert_offsets": offsets, "sorted_pairs": sorted_pairs,
            "pair_rows": pair_rows, "dropped": P - n}


# ----------------------------------------------------------------------------- quant


def _u16(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return np.asarray(x, dtype=np.uint16)


def quant_act_ref(x) -> tuple:
    """Online FP8 activation quantization ("Pushing the Limits of Serving
    DeepSeek-V4-Pro", §2.2): bf16 x [T, H] -> E4M3 codes [T, H] and one E8M0
    scale per token per 128 columns [T, H/128]."""
    codes, scales, _ = quantize_blocks(bf16_to_f64(_u16(x)), 128)
    return codes, scales


# ----------------------------------------------------------------------------- dequant

_E2M1_T = torch.from_numpy(E2M1_VALUES)
_E4M3_T = torch.from_numpy(E4M3_VALUES)
_E8M0_T = torch.from_numpy(E8M0_VALUES)
# value pair of one packed byte: (element 2i from the low nibble, element 2i+1 from the high)
_BYTE_PAIR = torch.stack([_E2M1_T[torch.arange(256) & 15], _E2M1_T[torch.arange(256) >> 4]], -1)


def dequant_mxfp4(codes, scales) -> torch.Tensor:
    """MXFP4 [N, K/2] codes + [N, K/32] E8M0 scales -> exact float64 [N, K]: each
    byte looked up as its (low nibble, high nibble) value pair, each 32-element
    block multiplied by its scale."""
    codes = torch.as_tensor(codes).cpu()
    scales = torch.as_tensor(scales).cpu()
    N, half = codes.shape
    w = _BYTE_PAIR.index_select(0, codes.reshape(-1).to(torch.int32)).view(N, half // 16, 32)
    return w.mul_(_E8M0_T[scales.to(torch.int64)].unsqueeze(-1)).view(N, 2 * half)


def dequant_nvfp4(codes, scales) -> torch.Tensor:
    """NVFP4 [N, K/2] codes + [N, K/16] E4M3 block scales -> exact float64 [N, K]
    without the tensor scale: each 16-element block times its E4M3 scale."""
    codes = torch.as_tensor(codes).cpu()
    scales = torch.as_tensor(scales).cpu()
    N, half = codes.shape
    w = _BYTE_PAIR.index_select(0, codes.reshape(-1).to(torch.int32)).view(N, half // 8, 16)
    return w.mul_(_E4M3_T[scales.to(torch.int64)].unsqueeze(-1)).view(N, 2 * half)


def dequant_fp8_block(codes, scales) -> torch.Tensor:
    """FP8 E4M3 [N, K] codes + [N/128, K/128] E8M0 block scales -> float64 [N, K]."""
    codes = torch.as_tensor(codes).cpu()
    scales = torch.as_tensor(scales).cpu()
    N, Kd = codes.shape
    v = _E4M3_T[codes.long()].reshape(N // 128, 128, Kd // 128, 128)
    return (v * _E8M0_T[scales.long()][:, None, :, None]).reshape(N, Kd)


def _silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def _expert_ffn(xh: torch.Tensor, W13: torch.Tensor, W2: torch.Tensor, I: int):
    """One expert on the dequantized rows xh [m, H] (float64): W13 GEMM, SwiGLU,
    requantization of the SwiGLU output, W2 GEMM. Returns (out [m, H] float64,
    h codes, h scale codes, h block amax)."""
    acc = (xh @ W13.T).numpy()
    g, u = acc[:, :I], acc[:, I:]
    h = _silu_mul(g, u)
    del acc, g, u
    hq, hs, amax = quantize_blocks(h, 128)
    hh = torch.from_numpy(dequantize_blocks(hq, hs, 128))
    return (hh @ W2.T).numpy(), hq, hs, amax


def _expert_ffn_a16(xh: torch.Tensor, W13: torch.Tensor, W2: torch.Tensor, I: int):
    """One expert with bf16 activations (MXFP4A16): W13 GEMM on the bf16 rows xh,
    SwiGLU, the SwiGLU output rounded to bf16, W2 GEMM on it. Returns (out [m, H]
    float64, h bf16 bit patterns [m, I])."""
    acc = (xh @ W13.T).numpy()
    hb = f64_to_bf16_rne(_silu_mul(acc[:, :I], acc[:, I:]))
    del acc
    return (torch.from_numpy(bf16_to_f64(hb)) @ W2.T).numpy(), hb


# ----------------------------------------------------------------------------- FFN


def ffn_ref(x, topk_ids, topk_weights, w13, w13_s, w2, w2_s, shared=None, tokens=None, act: str = "fp8") -> dict:
    """The routed MoE FFN in float64 for all tokens or for a subset ``tokens``.

    x bf16 [T, H]; topk_ids int [T, K]; topk_weights float32 [T, K]; w13 [E, 2I, H/2],
    w13_s [E, 2I, H/32], w2 [E, H, I/2], w2_s [E, H, I/32] (uint8, any device; the
    experts needed are copied to the host one at a time); ``shared`` = optional dict
    w13s [2Is, H], w13s_s [2Is/128, H/128], w2s [H, Is], w2s_s [H/128, Is/128].

    Returns dict with, for the selected tokens in the given order:
      y      float64 [n, H]
      x_q, x_s   activation codes / scales of those tokens
      h_q    uint8 [n, K, I]   SwiGLU-output codes per (token, pick)
      h_s    uint8 [n, K, I/128]
      h_amax float64 [n, K, I/128]
      valid  bool [n, K]       pick has an id in [0, E)
      shared_h_q / shared_h_s / shared_h_amax (when a shared expert is given).

    act="bf16" (MXFP4A16): x is not quantized; x_q / x_s are None, h_q holds the
    bf16 SwiGLU outputs (uint16 bit patterns [n, K, I]) and h_s / h_amax are None;
    no shared expert.

    Memory stays near one expert's working set: each expert's W2 outputs are
    added into y as soon as they are computed (the top-k reduction is a sum, so
    the order of its terms only moves float64 rounding), and no per-pair output
    rows are kept.
    """
    xb = _u16(x)
    ids = np.asarray(torch.as_tensor(topk_ids).cpu()).astype(np.int64)
    wts = np.asarray(torch.as_tensor(topk_weights).cpu()).astype(np.float64)
    T, H = xb.shape
    K = ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = sel.size
    if act not in ("fp8", "bf16"):
        raise ValueError(f"act must be 'fp8' or 'bf16', not {act!r}")
    if act == "bf16":
        if shared is not None:
            raise ValueError("the bf16-activation variant has no shared expert")
        return _ffn_ref_a16(xb[sel], ids[sel], wts[sel], w13, w13_s, w2, w2_s)

    x_q, x_s = quant_act_ref(xb[sel])
    xh = torch.from_numpy(dequantize_blocks(x_q, x_s, 128))

    y = np.zeros((n, H), dtype=np.float64)
    h_q = np.zeros((n, K, I), dtype=np.uint8)
    h_s = np.zeros((n, K, I // 128), dtype=np.uint8)
    h_amax = np.zeros((n, K, I // 128), dtype=np.float64)
    sid = ids[sel]
    valid = (sid >= 0) & (sid < E)
    for e in np.unique(sid[valid]):
        rows, picks = np.nonzero(sid == e)
        W13 = dequant_mxfp4(w13[int(e)], w13_s[int(e)])
        W2 = dequant_mxfp4(w2[int(e)], w2_s[int(e)])
        o, hq, hs, am = _expert_ffn(xh[torch.from_numpy(rows)], W13, W2, I)
        del W13, W2
        # top-k weighted reduction: a token may pick the same expert twice
        np.add.at(y, rows, wts[sel[rows], picks][:, None] * o)
        del o
        h_q[rows, picks] = hq
        h_s[rows, picks] = hs
        h_amax[rows, picks] = am
    res = {"y": y, "x_q": x_q, "x_s": x_s, "h_q": h_q, "h_s": h_s, "h_amax": h_amax,
           "valid": valid}
    if shared is not None:
        Is = shared["w2s"].shape[1]
        W13s = dequant_fp8_block(shared["w13s"], shared["w13s_s"])
        W2s = dequant_fp8_block(shared["w2s"], shared["w2s_s"])
        o, hq, hs, am = _expert_ffn(xh, W13s, W2s, Is)
        y += o
        res.update(shared_h_q=hq, shared_h_s=hs, shared_h_amax=am)
    return res


def _ffn_ref_a16(xb, sid, wts, w13, w13_s, w2, w2_s) -> dict:
    n, H = xb.shape
    K = sid.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    xh = torch.from_numpy(bf16_to_f64(xb))
    y = np.zeros((n, H), dtype=np.float64)
    h_q = np.zeros((n, K, I), dtype=np.uint16)
    valid = (sid >= 0) & (sid < E)
    for e in np.unique(sid[valid]):
        rows, picks = np.nonzero(sid == e)
        W13 = dequant_mxfp4(w13[int(e)], w13_s[int(e)])
        W2 = dequant_mxfp4(w2[int(e)], w2_s[int(e)])
        o, hb = _expert_ffn_a16(xh[torch.from_numpy(rows)], W13, W2, I)
        del W13, W2
        np.add.at(y, rows, wts[rows, picks][:, None] * o)
        h_q[rows, picks] = hb
    return {"y": y, "x_q": None, "x_s": None, "h_q": h_q, "h_s": None, "h_amax": None, "valid": valid}


def ffn_ref_nvfp4(x, topk_ids, topk_weights, w13, w13_s, w13_gs, w2, w2_s, w2_gs, tokens=None) -> dict:
    """The routed MoE FFN with NVFP4 expert weights and bf16 activations, float64,
    for all tokens or the subset ``tokens``. w13 [E, 2I, H/2] / w2 [E, H, I/2]
    codes, w13_s [E, 2I, H/16] / w2_s [E, H, I/16] E4M3 block scales, w13_gs /
    w2_gs [E] tensor scales. Per expert e:
        g, u = gs13[e] * (x . W13'[e]^T) split at I   (W' = codes x block scales)
        h    = bf16(silu(g) * u)
        o    = gs2[e] * (h . W2'[e]^T)
    and y = sum_j w[t, j] o. Returns y, h_q (bf16 bits [n, K, I]), valid."""
    xb = _u16(x)
    ids = np.asarray(torch.as_tensor(topk_ids).cpu()).astype(np.int64)
    wts = np.asarray(torch.as_tensor(topk_weights).cpu()).astype(np.float64)
    gs13 = np.asarray(torch.as_tensor(w13_gs).cpu()).astype(np.float64)
    gs2 = np.asarray(torch.as_tensor(w2_gs).cpu()).astype(np.float64)
    T, H = xb.shape
    K = ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    sel = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = sel.size
    sid = ids[sel]
    xh = torch.from_numpy(bf16_to_f64(xb[sel]))
    y = np.zeros((n, H), dtype=np.float64)
    h_q = np.zeros((n, K, I), dtype=np.uint16)
    valid = (sid >= 0) & (sid < E)
    for e in np.unique(sid[valid]):
        rows, picks = np.nonzero(sid == e)
        acc = (xh[torch.from_numpy(rows)] @ dequant_nvfp4(w13[int(e)], w13_s[int(e)]).T).numpy() * gs13[e]
        hb = f64_to_bf16_rne(_silu_mul(acc[:, :I], acc[:, I:]))
        del acc
        o = (torch.from_numpy(bf16_to_f64(hb)) @ dequant_nvfp4(w2[int(e)], w2_s[int(e)]).T).numpy() * gs2[e]
        np.add.at(y, rows, wts[sel[rows], picks][:, None] * o)
        h_q[rows, picks] = hb
    return {"y": y, "h_q": h_q, "valid": valid}


def ffn_ref_dense_single(x, w13, w13_s, w2, w2_s) -> np.ndarray:
    """A single MXFP4 SwiGLU expert applied densely to every token (no routing):
    the special case K = 1 / E = 1 of ``ffn_ref`` with weight 1. Written as plain
    matrix products over all tokens at once."""
    xq, xs = quant_act_ref(x)
    xh = torch.from_numpy(dequantize_blocks(xq, xs, 128))
    I = w2.shape[1] * 2
    o = _expert_ffn(xh, dequant_mxfp4(w13, w13_s), dequant_mxfp4(w2, w2_s), I)[0]
    return o
