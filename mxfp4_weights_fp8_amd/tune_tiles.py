"""Exact-shape tiling sweep: for a workload's routing histogram, time the W13 and W2
stages with each choice of how many rows a 128-row work item (an expert's remainder
of 1..128 rows, or a whole expert of at most 128 pairs) may have and still run as
16-row small-M tiles instead of one 128-row large-M tile (moe_dims.tile_w13 /
tile_w2), and report the fastest choice per GEMM. Its output is what the library's
table of (H, I) -> (tile_w13, tile_w2) holds.

    python -m mxfp4_weights_fp8_amd.tune_tiles [--workloads prefill32k,tp8rank32k] [--steps 5]

Needs a GPU; the synthetic workloads come from synth/. Times are medians over
steps of HIP events the library records around each stage, averaged over rounds
that visit the candidates in alternating order after a warm-up pass.
"""

from __future__ import annotations

import argparse
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import mxfp4_weights_fp8_amd as moe  # noqa: E402
from synth import WORKLOADS, make_expert_weights, make_inputs, make_shared_weights  # noqa: E402

CANDIDATES = (-1, 16, 32, 48, 64, 80, 96, 112, 128)


def remainder_histogram(ids: np.ndarray, E: int, small_max: int = 16):
    """Rows of the 128-row items the planner makes for this routing."""
    m = np.bincount(ids[(ids >= 0) & (ids < E)].ravel(), minlength=E)
    r = m % 256
    return np.sort(r[(m > small_max) & (r >= 1) & (r <= 128)])


def sweep(name: str, steps: int, dev, weights=None, rounds: int = 3):
    w = WORKLOADS[name]
    inp = make_inputs(name, weights=False).to(dev)
    W = weights if weights is not None else moe.pack_weights(make_expert_weights(w, dev))
    sh = make_shared_weights(w, dev) if w.Is else None
    rem = remainder_histogram(inp.topk_ids.cpu().numpy(), w.E)
    print(f"[{name}] {rem.size} items of 1..128 rows; rows quantiles 10/50/90%: "
          f"{np.quantile(rem, [0.1, 0.5, 0.9]).round(1).tolist() if rem.size else []}", flush=True)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    runs = {}
    for t in CANDIDATES:
        p = moe.plan(inp.topk_ids, w.E, w.H, w.I, Is=w.Is, tile_w13=t, tile_w2=t)
        ws = torch.empty(moe.ffn_workspace_bytes(p.dims), dtype=torch.uint8, device=dev)
        runs[t] = (p, ws)

    def measure(t):
        p, ws = runs[t]

        def step(ev=None):
            moe.plan(inp.topk_ids, w.E, w.H, w.I, Is=w.Is, out=p, tile_w13=t, tile_w2=t)
            moe.ffn(inp.x, inp.topk_weights, p, W, shared=sh, ws=ws, y=y, events=ev)

        step()
        evs = [moe.StageEvents() for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        med = lambda a, b: float(np.median([e.elapsed_ms(a, b) for e in evs]))
        return (med(moe.EV_QUANT_DONE, moe.EV_W13_DONE), med(moe.EV_W13_DONE, moe.EV_W2_DONE),
                med(moe.EV_START, moe.EV_END))

    # one warm-up pass over every candidate, then rounds in alternating order (the
    # first configuration measured after a change of work runs a few percent slow)
    for t in CANDIDATES:
        measure(t)
    samples = {t: [] for t in CANDIDATES}
    for r in range(rounds):
        for t in (CANDIDATES if r % 2 == 0 else CANDIDATES[::-1]):
            samples[t].append(measure(t))
    res = {}
    for t in CANDIDATES:
        a = np.array(samples[t])
        res[t] = tuple(a.mean(axis=0))
        n_small = int((rem <= t).sum()) if t > 0 else 0
        print(f"[{name}] tile {t:4d}: {n_small:3d} items small; W13 {res[t][0]:.4f} ms (spread "
              f"{np.ptp(a[:, 0]):.4f})  W2 {res[t][1]:.4f} ms (spread {np.ptp(a[:, 1]):.4f})  ffn {res[t][2]:.4f} ms",
              flush=True)
    del runs
    b13 = min(res, key=lambda t: res[t][0])
    b2 = min(res, key=lambda t: res[t][1])
    print(f"[{name}] best: tile_w13 {b13} (W13 {res[b13][0]:.4f} vs {res[-1][0]:.4f} ms with none), "
          f"tile_w2 {b2} (W2 {res[b2][1]:.4f} vs {res[-1][1]:.4f} ms); table entry H {w.H} I {w.I}: "
          f"{{{w.H}, {w.I}, {max(b13, 0)}, {max(b2, 0)}}}", flush=True)
    return res, b13, b2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="prefill32k,tp8rank32k")
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--rounds", type=int, default=3)
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    moe.lib()
    full = None
    for name in args.workloads.split(","):
        w = WORKLOADS[name]
        shared_set = (w.H, w.I, w.E) == (7168, 3072, 384) and not w.full_I
        if shared_set and full is None:
            full = moe.pack_weights(make_expert_weights(WORKLOADS["decode7"], dev))
        sweep(name, args.steps, dev, full if shared_set else None, args.rounds)


if __name__ == "__main__":
    main()
