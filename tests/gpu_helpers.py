"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding, run the oracle on the same seeded inputs, compare."""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import mxfp4_weights_fp8_amd as moe
from oracle.compare import h_bf16_mismatch, h_code_mismatch, y_metrics
from oracle.formats import bf16_to_f64
from oracle.envelope import (routed_swiglu_envelope, routed_swiglu_envelope_a16, routed_swiglu_envelope_nvfp4,
                             shared_swiglu_envelope)
from oracle.moe import ffn_ref, ffn_ref_nvfp4, plan_ref

#: the parity bar for the final output (vs the float64 oracle)
MAX_REL = 2e-2
MEAN_REL = 2e-3
#: SwiGLU-output codes (routed and shared): at most this fraction may differ from
#: the oracle's, each by one grid step (or a scale flip at a boundary)
H_DIFFER = 1e-3
#: codes more than one step away must round from inside the hardware-dot envelope
#: (oracle/envelope.py), and at most this many may exist: max(2, 2e-5 of the codes)
BEYOND_FRAC = 2e-5
#: bf16 SwiGLU outputs (bf16-activation variant): every difference from the oracle
#: must round from inside the hardware-dot envelope; as a coarse guard on top, at
#: most this fraction may differ at all (a one-step bf16 difference needs the fp32
#: SwiGLU value within the envelope of a rounding boundary: about 2 * err / ulp of
#: the elements, err / ulp near 1e-3 .. 1e-2 on these workloads)
H16_DIFFER = 2e-2


def beyond_cap(n: int) -> int:
    return max(2, int(np.ceil(BEYOND_FRAC * n)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_path(inp, small_max=0, debug=True, flags=0):
    """plan + ffn on the GPU for MoEInputs already on the device. The workspace and
    y start as 0xFF bytes (NaN as fp16 and bf16), so a row that no kernel writes
    shows up in the comparison with the oracle instead of passing on stale data."""
    w = inp.wl
    p = moe.plan(inp.topk_ids, w.E, w.H, w.I, small_max=small_max, Is=w.Is if inp.shared else 0, flags=flags)
    packed = moe.pack_weights(inp.weights)
    ws = torch.full((moe.ffn_workspace_bytes(p.dims),), 0xFF, dtype=torch.uint8, device=inp.x.device)
    y = torch.full((w.T, w.H), -1, dtype=torch.int16, device=inp.x.device).view(torch.bfloat16)
    out = moe.ffn(inp.x, inp.topk_weights, p, packed, shared=inp.shared, debug=debug, ws=ws, y=y)
    del packed
    torch.cuda.synchronize()
    return p, out


def check_plan(p, ids_np, E):
    ref = plan_ref(ids_np, E)
    P = ids_np.size
    assert np.array_equal(p.expert_offsets.cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(p.sorted_pairs.cpu().numpy()[:P], ref["sorted_pairs"])
    assert np.array_equal(p.pair_rows.cpu().numpy()[:P], ref["pair_rows"])
    assert int(p.status.cpu()[0]) == ref["dropped"]


def _host(t):
    return t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def routed_envelope(inp, ref, sel, pairs):
    """Envelope callback for the routed SwiGLU codes compared in pair order
    ``pairs`` (list of (token position in sel, pick)): exact values and bounds,
    one expert's row-major W13 copied to the host at a time."""
    ids = _host(inp.topk_ids)
    W = inp.weights
    I = inp.wl.I

    def f(rows, cols):
        h = np.zeros(rows.size)
        err = np.zeros(rows.size)
        tpos = np.array([pairs[r][0] for r in rows])
        exp = np.array([ids[sel[pairs[r][0]], pairs[r][1]] for r in rows])
        for e in np.unique(exp):
            m = exp == e
            w13 = _host(W["w13"][int(e)])
            w13_s = _host(W["w13_s"][int(e)])
            h[m], err[m] = routed_swiglu_envelope(ref["x_q"], ref["x_s"], w13, w13_s, I, tpos[m], cols[m])
        return h, err
    return f


def shared_envelope(inp, ref):
    sh = {k: _host(v) for k, v in inp.shared.items()}

    def f(rows, cols):
        return shared_swiglu_envelope(ref["x_q"], ref["x_s"], sh["w13s"], sh["w13s_s"], inp.wl.Is, rows, cols)
    return f


def check_codes(m: dict, prefix: str):
    """The SwiGLU-code bar on a comparison from h_code_mismatch."""
    n = m[prefix + "elements"]
    assert m[prefix + "bad"] == 0, m
    assert m[prefix + "frac_differ"] <= H_DIFFER, m
    assert m[prefix + "beyond"] <= beyond_cap(n), m


_SUMMED = ("elements", "differ", "one_step", "scale_flip", "beyond", "in_envelope", "bad", "scale_diff_blocks")


def codes_chunked(get_gpu, hq_ref, hs_ref, amax_ref, envelope, rows_per_chunk: int = 16384) -> dict:
    """h_code_mismatch over row chunks (bounded host memory at full sizes), counts
    summed. get_gpu(r0, r1) -> (hq, hs) of compared rows r0..r1; envelope rows are
    global row indices."""
    R = hq_ref.shape[0]
    tot = {k: 0 for k in _SUMMED}
    tot["max_code_dist_same_scale"] = 0
    tot["bad_examples"] = []
    for r0 in range(0, max(R, 1), rows_per_chunk):
        r1 = min(R, r0 + rows_per_chunk)
        if r1 <= r0:
            break
        hq, hs = get_gpu(r0, r1)
        env = None if envelope is None else (lambda rows, cols, r0=r0: envelope(rows + r0, cols))
        m = h_code_mismatch(hq, hs, hq_ref[r0:r1], hs_ref[r0:r1], amax_ref[r0:r1], envelope=env)
        for k in _SUMMED:
            tot[k] += m[k]
        tot["max_code_dist_same_scale"] = max(tot["max_code_dist_same_scale"], m["max_code_dist_same_scale"])
        tot["bad_examples"] += m["bad_examples"][:5 - len(tot["bad_examples"])]
    tot["frac_differ"] = tot["differ"] / max(tot["elements"], 1)
    return tot


def check_ffn(inp, p, y, dbg, tokens=None, label="", ref=None):
    """Oracle on the selected tokens; compare y, x codes, SwiGLU codes. Returns metrics.
    ``ref``: a precomputed ffn_ref result for these tokens (else it is computed)."""
    t0 = time.time()
    if ref is None:
        ref = ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **inp.weights, shared=inp.shared, tokens=tokens)
    t_oracle = time.time() - t0
    sel = np.arange(inp.wl.T) if tokens is None else np.asarray(tokens)
    yb = u16(y)[sel]
    m = y_metrics(yb, ref["y"])
    # activation codes: bit-exact
    assert np.array_equal(dbg["x_q"].cpu().numpy()[sel], ref["x_q"]), "x_q differs"
    assert np.array_equal(dbg["x_s"].cpu().numpy()[sel], ref["x_s"]), "x_s differs"
    # SwiGLU codes of every valid pick of the selected tokens, rows in plan order
    K = inp.wl.K
    valid = ref["valid"]
    rows = p.pair_rows.cpu().numpy()
    vi, vj = np.nonzero(valid)
    pairs = list(zip(vi.tolist(), vj.tolist()))
    prow = torch.from_numpy(rows[sel[vi] * K + vj].astype(np.int64))

    def gpu_rows(r0, r1):
        idx = prow[r0:r1].to(dbg["h_q"].device)
        return dbg["h_q"][idx].cpu().numpy(), dbg["h_s"][idx].cpu().numpy()

    hm = codes_chunked(gpu_rows, ref["h_q"][valid], ref["h_s"][valid], ref["h_amax"][valid],
                       routed_envelope(inp, ref, sel, pairs))
    m.update({"h_" + k: v for k, v in hm.items()}, oracle_s=round(t_oracle, 2), label=label)
    if inp.shared is not None:
        Is = inp.wl.Is
        shq = dbg["sh_q"].cpu().numpy()[sel][:, :Is]
        shs = dbg["sh_s"].cpu().numpy()[sel][:, :Is // 128]
        shm = codes_chunked(lambda r0, r1: (shq[r0:r1], shs[r0:r1]), ref["shared_h_q"], ref["shared_h_s"],
                            ref["shared_h_amax"], shared_envelope(inp, ref))
        m.update({"sh_" + k: v for k, v in shm.items()})
    say(f"[parity {label}] {m}")
    assert m["finite"], m
    if m["max_rel"] > MAX_REL:
        yv = bf16_to_f64(yb)
        err = np.abs(yv - ref["y"]).max(axis=-1) / np.abs(ref["y"]).max()
        worst = np.argsort(-err)[:8]
        rows = []
        for i in worst:
            bad_cols = np.nonzero(np.abs(yv[i] - ref["y"][i]) > MAX_REL * np.abs(ref["y"]).max())[0]
            rows.append((int(sel[i]), float(err[i]), int(bad_cols.size), bad_cols[:8].tolist(),
                         inp.topk_ids[int(sel[i])].tolist()))
        say(f"[parity {label}] worst rows (token, rel err, bad columns, first columns, experts): {rows}")
    assert m["max_rel"] <= MAX_REL, m
    assert m["mean_rel"] <= MEAN_REL, m
    check_codes(m, "h_")
    if inp.shared is not None:
        check_codes(m, "sh_")
    return m


def check_ffn_a16(inp, p, y, dbg, tokens=None, label="", ref=None, nvfp4=False):
    """The bf16-activation variants (MXFP4 weights: oracle act="bf16"; nvfp4=True:
    NVFP4 weights, ffn_ref_nvfp4, with inp.weights the row-major NVFP4 tensors) on
    the selected tokens; compare y and every valid pick's bf16 SwiGLU outputs.
    Returns metrics."""
    t0 = time.time()
    if ref is None:
        if nvfp4:
            ref = ffn_ref_nvfp4(inp.x, inp.topk_ids, inp.topk_weights, **inp.weights, tokens=tokens)
        else:
            ref = ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **inp.weights, tokens=tokens, act="bf16")
    t_oracle = time.time() - t0
    sel = np.arange(inp.wl.T) if tokens is None else np.asarray(tokens)
    yb = u16(y)[sel]
    m = y_metrics(yb, ref["y"])
    K, I = inp.wl.K, inp.wl.I
    valid = ref["valid"]
    rows = p.pair_rows.cpu().numpy()
    vi, vj = np.nonzero(valid)
    prow = torch.from_numpy(rows[sel[vi] * K + vj].astype(np.int64))
    hg = u16(dbg["h_q"][prow.to(dbg["h_q"].device)]) if prow.numel() else np.zeros((0, I), np.uint16)
    ids = _host(inp.topk_ids)
    xb = u16(inp.x)[sel]
    W = inp.weights

    def envelope(r, c):
        h = np.zeros(r.size)
        err = np.zeros(r.size)
        exp = ids[sel[vi[r]], vj[r]]
        for e in np.unique(exp):
            mk = exp == e
            if nvfp4:
                h[mk], err[mk] = routed_swiglu_envelope_nvfp4(xb, _host(W["w13"][int(e)]), _host(W["w13_s"][int(e)]),
                                                              float(W["w13_gs"][int(e)]), I, vi[r][mk], c[mk])
            else:
                h[mk], err[mk] = routed_swiglu_envelope_a16(xb, _host(W["w13"][int(e)]), _host(W["w13_s"][int(e)]),
                                                            I, vi[r][mk], c[mk])
        return h, err

    hm = h_bf16_mismatch(hg, ref["h_q"][valid], envelope=envelope)
    m.update({"h_" + k: v for k, v in hm.items()}, oracle_s=round(t_oracle, 2), label=label)
    say(f"[parity {'nvfp4' if nvfp4 else 'a16'} {label}] {m}")
    assert m["finite"], m
    assert m["max_rel"] <= MAX_REL, m
    assert m["mean_rel"] <= MEAN_REL, m
    assert m["h_bad"] == 0, m
    assert m["h_frac_differ"] <= H16_DIFFER, m
    return m
