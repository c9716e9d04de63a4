"""Benchmark of the routed MoE FFN (MXFP4 weights, FP8 activations) on one MI355X.

A step is one pass of the whole hot path over one batch resident in HBM: route
plan (moe_plan) + activation quantization, W13 GEMM with the fused SwiGLU + FP8
requantization, W2 GEMM and the top-k combine (moe_ffn).

The headline line is the 7-token decode verify (H 7168, 384 experts, I 3072,
top-8, Zipf 1.0 routing): tokens/s, with the roofline of its dominant kernel
(the W13 weight stream, HBM-bound). The same JSON line carries the 256-token
decode step (32 requests x 8 positions) as "decode256" (HBM roofline), the
32K-token prefill chunk (Zipf 1.2) as "prefill32k" (MFMA roofline of its W13
GEMM) and one MoE-TP8 rank of it as "tp8rank32k" (MFMA and HBM bounds), because
the metric names them; "decode7_a16" and "decode256_a16" time the two decode
steps with bf16 activations (the MXFP4A16 variant, MOE_FLAG_A16), and
"decode7_nvfp4" / "decode256_nvfp4" with NVFP4 expert weights (moe_ffn_nvfp4).
Kernel durations come from HIP events the library records on the stream it
launches on (in the decode objects on every 4th timed step: an event record costs
about 3 us of stream time); the oracle's CPU time on bounded samples is reported
as cpu_baseline. The prefill objects also time the vendor library's dense FP8
GEMM on each GEMM's total shape (``dense_fp8_gemm_reference``), as a practical
reference for the MFMA fraction.

Every workload is timed twice: back-to-back steps (the contract's timed region,
``ms_per_step``), and steps each preceded by a 1 GiB read that evicts the
256 MB last-level cache, timed one by one with events (``mall_flushed``), so the
HBM figures cannot include last-level-cache hits from the previous step. The
flush reads rather than writes: a written flush leaves up to 256 MB of dirty
lines whose write-back would be charged to the next step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mxfp4_weights_fp8_amd as moe  # noqa: E402
from synth import WORKLOADS, make_expert_weights, make_inputs, make_shared_weights  # noqa: E402

METRIC = "MoE FFN tokens/s + % MFMA peak (32K prefill) + HBM GB/s (decode M=7)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_FP8_TFLOPS = 5000.0  # dense FP8 rate; a block-scaled MFMA with one 8-bit operand issues at it
MFMA_PEAK_FP4_TFLOPS = 10100.0 # dense FP4/FP6 rate (both operands <= 6 bits)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(w, nvfp4: bool = False) -> dict:
    """Algorithmic bytes of one expert's 4-bit weights: MXFP4 codes + E8M0 scales
    per 32, or NVFP4 codes + E4M3 scales per 16 + one fp32 tensor scale."""
    H, I = w.H, w.I
    blk, extra = (16, 4) if nvfp4 else (32, 0)
    w13 = 2 * I * H // 2 + 2 * I * H // blk + extra
    w2 = H * I // 2 + H * I // blk + extra
    return {"w13": w13, "w2": w2}


def measured_traffic(workload: str, kernels):
    """HBM bytes per launch of the given kernels together (one name or a list: a
    stage made of several launches) from the committed rocprofv3 counter summary
    of ``workload`` (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known
    size), or None when there is no summary, a kernel is missing from it, or a
    kernel's sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    names = [kernels] if isinstance(kernels, str) else list(kernels)
    found = {}
    for line in open(path):
        if line.startswith("#"):
            continue
        f = line.strip().rsplit(",", 6)   # kernel names may hold commas (template arguments)
        if len(f) == 7 and f[0] in names and f[5] != "-":
            h = hashlib.sha256()
            for name in f[5].split("+"):
                h.update(open(os.path.join(ROOT, "mxfp4_weights_fp8_amd", "csrc", name), "rb").read())
            if h.hexdigest() != f[6]:
                return None
            found[f[0]] = float(f[4])
    return sum(found.values()) if len(found) == len(names) else None


class Runner:
    """Holds one workload resident on the GPU and runs steps of the hot path."""

    def __init__(self, name: str, dev, weights=None, flags: int = 0):
        """weights: expert weights already converted with moe.pack_weights (None:
        generate and convert this workload's own); flags: moe_dims flags."""
        self.w = WORKLOADS[name]
        w = self.w
        inp = make_inputs(name, weights=False).to(dev)
        inp.weights = weights if weights is not None else moe.pack_weights(make_expert_weights(w, dev))
        inp.shared = make_shared_weights(w, dev) if w.Is else None
        self.inp = inp
        self.dev = dev
        self.flags = flags
        self.plan = moe.plan(inp.topk_ids, w.E, w.H, w.I, Is=w.Is, flags=flags)
        d = self.plan.dims
        self.ws = torch.empty(moe.ffn_workspace_bytes(d), dtype=torch.uint8, device=dev)
        self.y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
        ids = inp.topk_ids.cpu().numpy()
        self.distinct = int(len(np.unique(ids[(ids >= 0) & (ids < w.E)])))

    def step(self, events=None):
        w = self.w
        moe.plan(self.inp.topk_ids, w.E, w.H, w.I, Is=w.Is, out=self.plan, flags=self.flags)
        moe.ffn(self.inp.x, self.inp.topk_weights, self.plan, self.inp.weights, shared=self.inp.shared,
                ws=self.ws, y=self.y, events=events)

    def run(self, steps: int, warmup: int, focus=(moe.EV_QUANT_DONE, moe.EV_W13_DONE), every: int = 1):
        """Warmup, then `steps` timed steps. In every `every`-th timed step (from the
        first) the library records the two events around the focus stage, and only
        those: each event record costs about 3 us of stream time (decode7: 0.2274
        ms per step with the events on every step, 0.2222 on every 4th, 0.2210 with
        none, one box). Returns (ms per step, focus stage ms averaged over the timed
        steps that recorded it, per-stage ms from a separate untimed pass with every
        stage event)."""
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [moe.StageEvents(only=focus) if i % every == 0 else None for i in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        self.focus_launches = sum(e is not None for e in evs)
        focus_ms = float(np.mean([e.elapsed_ms(*focus) for e in evs if e is not None]))
        diag = [moe.StageEvents() for _ in range(max(3, min(steps, 10)))]
        for e in diag:
            self.step(e)
        torch.cuda.synchronize()
        stages = {"quant": (moe.EV_START, moe.EV_QUANT_DONE), "w13": (moe.EV_QUANT_DONE, moe.EV_W13_DONE),
                  "w2": (moe.EV_W13_DONE, moe.EV_W2_DONE), "shared": (moe.EV_W2_DONE, moe.EV_SHARED_DONE),
                  "combine": (moe.EV_SHARED_DONE, moe.EV_END), "ffn": (moe.EV_START, moe.EV_END)}
        ms = {k: float(np.mean([e.elapsed_ms(a, b) for e in diag])) for k, (a, b) in stages.items()}
        return (t1 - t0) * 1e3 / steps, focus_ms, ms

    def run_flushed(self, steps: int, flush: torch.Tensor, focus=(moe.EV_QUANT_DONE, moe.EV_W13_DONE)):
        """`steps` steps, each after a read of `flush` (1 GiB of clean lines that
        evict the 256 MB last-level cache), outside the events that time the step
        (plan + FFN) and the focus stage. Returns (median ms per step, median
        focus-stage ms, largest step ms): steps are timed one by one, and the median
        keeps a rare stalled step (one of 50 took tens of ms once) from moving the
        figure."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                moe.StageEvents(only=focus)) for _ in range(steps)]
        for i, (a, b, st) in enumerate(evs):
            flush.max()
            a.record()
            self.step(st)
            b.record()
        torch.cuda.synchronize()
        step_ms = [a.elapsed_time(b) for a, b, _ in evs]
        return (float(np.median(step_ms)), float(np.median([st.elapsed_ms(*focus) for _, _, st in evs])),
                float(np.max(step_ms)))


def cpu_baseline(name: str, weights_dev, tokens) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload's tokens.
    weights_dev: the row-major expert weights on the device; the experts those
    tokens use are copied to host memory before the clock starts."""
    from oracle.moe import ffn_ref

    inp = make_inputs(name, weights=False)
    ids = inp.topk_ids.numpy()[tokens]
    used = sorted(set(int(e) for e in ids.ravel() if 0 <= e < inp.wl.E))
    host = {k: torch.empty(v.shape, dtype=v.dtype) for k, v in weights_dev.items()}   # untouched rows unused
    for k, v in weights_dev.items():
        host[k][used] = v[used].cpu()
    t0 = time.perf_counter()
    ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **host, tokens=tokens)
    dt = time.perf_counter() - t0
    return {"value": len(tokens) / dt, "unit": "tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{len(tokens)} of {inp.wl.T} tokens of {name} (float64 oracle incl. expert dequant), "
                      f"{dt:.1f} s"}


# The decode objects time their dominant launch with events on every 4th timed step:
# the other steps run as a caller would run them, with no event records.
DECODE_EVENT_EVERY = 4
CHAIN_MAX_PAIRS = 512   # up to this many pairs MOE_FLAG_DECODE_CHAIN runs W13, W2 and the combine as one launch


def decode_object(r: Runner, steps: int, warmup: int, flush: torch.Tensor) -> dict:
    """A decode workload: tokens/s, the HBM roofline of its dominant launch (the
    weight stream of every touched expert), the whole step's HBM rate, and the same
    with the last-level cache flushed before each step.

    With MOE_FLAG_DECODE_CHAIN (up to CHAIN_MAX_PAIRS pairs) the dominant launch is
    the persistent decode chain (W13 + SwiGLU/requant, W2 and the combine): its
    algorithmic bytes are both weight sets of every touched expert, the activation
    codes read and y written, and its time the span between the stage events around
    it. Otherwise it is the W13 stage (W13 weights, activation codes, SwiGLU codes
    written); with MOE_FLAG_A16 (bf16 activations) the activations read and the
    SwiGLU rows written are bf16, 2 bytes per element and no scales."""
    w = r.w
    P = w.T * w.K
    nv = bool(r.flags & moe.FLAG_NVFP4)
    a16 = bool(r.flags & (moe.FLAG_A16 | moe.FLAG_NVFP4))
    chain = bool(r.flags & moe.FLAG_DECODE_CHAIN) and P <= CHAIN_MAX_PAIRS and not a16
    ms_step, dom_ms, stages = r.run(steps, warmup, every=DECODE_EVENT_EVERY)
    fl_step, fl_dom, fl_max = r.run_flushed(steps, flush)
    eb = expert_bytes(w, nvfp4=nv)
    if chain:
        dom_bytes = r.distinct * (eb["w13"] + eb["w2"]) + w.T * (w.H + w.H // 128) + w.T * w.H * 2
        dom_name = "decode chain: W13 + SwiGLU/requant, W2, combine in one launch (k_decode_chain)"
        traffic = measured_traffic(w.name + "_chain", "moe::k_decode_chain")
    elif a16:
        dom_bytes = r.distinct * eb["w13"] + w.T * w.H * 2 + P * w.I * 2
        # the kernel's second template argument is its wave count: MXFP4 4; NVFP4 8 up to
        # 512 pairs, 4 above
        kname = "k_w13_a16<true, %d>" % (8 if P <= 512 else 4) if nv else "k_w13_a16<false, 4>"
        dom_name = ("W13 stage, NVFP4 weights, bf16 activations: grouped GEMM + SwiGLU (%s)" if nv else
                    "W13 stage, bf16 activations: grouped GEMM + SwiGLU (%s)") % kname
        # one dispatch per step up to 128 pairs (above, a second one walks the 256-row
        # items, and the per-dispatch counter average no longer is the stage's traffic)
        traffic = (measured_traffic(w.name + ("_nvfp4" if nv else "_a16"), "moe::" + kname)
                   if P <= 128 else None)
    else:
        dom_bytes = r.distinct * eb["w13"] + w.T * (w.H + w.H // 128) + P * (w.I + w.I // 128)
        dom_name = "W13 stage: grouped GEMM + SwiGLU/requant (k_w13_small<4>" + \
            (" + large-M tiles)" if P > CHAIN_MAX_PAIRS else ")")
        # at most 512 pairs the stage is one launch; above, the small-M launch plus the
        # 256-row and 128-row launches (one dispatch each per step)
        traffic = measured_traffic(w.name, "moe::k_w13_small<4>" if P <= CHAIN_MAX_PAIRS else
                                   ["moe::k_w13_small<4>", "moe::k_gemm_xl<true>", "moe::k_gemm_large<true>"])
    # whole step: both weight sets of every touched expert, x in and y out (bf16)
    step_bytes = r.distinct * (eb["w13"] + eb["w2"]) + w.T * w.H * 2 * 2
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    log(f"[bench] {w.name}: {ms_step:.4f} ms/step ({fl_step:.4f} flushed), dominant launch {dom_ms:.4f} ms "
        f"({fl_dom:.4f} flushed), distinct experts {r.distinct}, stages {stages}")
    return {
        "value": w.T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step, "steps": steps,
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "intermediate": w.I,
                   "top_k": w.K, "routing": w.routing + f" s={w.zipf_s}", "distinct_experts": r.distinct,
                   **({"weights": "NVFP4 (E4M3 per 16 + fp32 tensor scale)", "activations": "bf16"} if nv else
                      {"activations": "bf16 (MXFP4A16)"} if a16 else {})},
        "roofline": {"bound": "hbm", "kernel": dom_name,
                     "achieved": gbs(dom_bytes, dom_ms), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs(dom_bytes, dom_ms) / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": dom_ms,
                     "launches_timed": f"{r.focus_launches} of the {steps} timed steps (HIP events on the "
                                       f"library's stream, every {DECODE_EVENT_EVERY}th step)"},
        "step_hbm_gbs": gbs(step_bytes, ms_step), "step_hbm_frac": gbs(step_bytes, ms_step) / HBM_PEAK_GBS,
        "step_algorithmic_bytes": step_bytes,
        "mall_flushed": {"ms_per_step": fl_step, "max_ms_per_step": fl_max, "value": w.T / (fl_step * 1e-3),
                         "dominant_ms": fl_dom,
                         "dominant_hbm_frac": gbs(dom_bytes, fl_dom) / HBM_PEAK_GBS,
                         "step_hbm_frac": gbs(step_bytes, fl_step) / HBM_PEAK_GBS},
        "stage_ms_untimed_pass": stages,
    }


def dense_fp8_reference(M: int, N: int, K: int, dev, reps: int = 10) -> dict:
    """The vendor library's dense FP8 GEMM (hipBLASLt through torch._scaled_mm: E4M3
    operands, one scale per tensor, bf16 out) on the dense problem of the same total
    shape, M rows x N outputs x K: no gather, no block scales, no fused epilogue, no
    expert boundaries. Context for the MFMA fraction (what a tuned dense GEMM
    reaches on this part at this shape), never part of a step."""
    a = torch.randn((M, K), dtype=torch.bfloat16, device=dev).to(torch.float8_e4m3fn)
    b = torch.randn((N, K), dtype=torch.bfloat16, device=dev).to(torch.float8_e4m3fn)
    one = torch.ones((), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch._scaled_mm(a, b.t(), one, one, out_dtype=torch.bfloat16, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch._scaled_mm(a, b.t(), one, one, out_dtype=torch.bfloat16, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    del a, b, out
    torch.cuda.empty_cache()
    return {"shape_MNK": [M, N, K], "ms": ms, "tflops": tf, "frac_fp8_peak": tf / MFMA_PEAK_FP8_TFLOPS}


def prefill_object(r: Runner, steps: int, flush: torch.Tensor) -> dict:
    """A prefill workload: tokens/s, the MFMA roofline of its W13 stage, the whole
    step against both the MFMA and the HBM bound, and the cache-flushed times."""
    w = r.w
    ps, p13_ms, stages = r.run(steps, 2)
    fl_step, fl_w13, fl_max = r.run_flushed(steps, flush)
    P = w.T * w.K
    f13 = 2.0 * P * (2 * w.I) * w.H
    f2 = 2.0 * P * w.H * w.I
    fs = (2.0 * w.T * (2 * w.Is) * w.H + 2.0 * w.T * w.H * w.Is) if w.Is else 0.0
    flops = f13 + f2 + fs
    eb = expert_bytes(w)
    # algorithmic bytes of the step: every expert's weights once, the shared expert's
    # FP8 weights + scales, x in and y out (bf16)
    shared_bytes = (3 * w.Is * w.H + 3 * w.Is * w.H // (128 * 128)) if w.Is else 0
    step_bytes = r.distinct * (eb["w13"] + eb["w2"]) + shared_bytes + w.T * w.H * 2 * 2
    t13 = f13 / (p13_ms * 1e-3) / 1e12
    tstep = flops / (ps * 1e-3) / 1e12
    ref13 = dense_fp8_reference(P, 2 * w.I, w.H, r.dev)
    ref2 = dense_fp8_reference(P, w.H, w.I, r.dev)
    t2 = f2 / (stages["w2"] * 1e-3) / 1e12
    log(f"[bench] {w.name}: {ps:.3f} ms/step ({fl_step:.3f} flushed), w13 {p13_ms:.3f} ms, stages {stages}; "
        f"dense FP8 GEMM of the same shapes: W13 {ref13['tflops']:.0f} TFLOP/s, W2 {ref2['tflops']:.0f} TFLOP/s")
    return {
        "value": w.T / (ps * 1e-3), "unit": "tokens/s", "ms_per_step": ps, "steps": steps,
        "config": {"workload": w.name, "tokens": w.T, "intermediate": w.I, "shared_intermediate": w.Is,
                   "routing": f"zipf s={w.zipf_s}"},
        "effective_tflops": tstep,
        "mfma_frac_fp8_peak": tstep / MFMA_PEAK_FP8_TFLOPS,
        "roofline": {"bound": "mfma",
                     "kernel": "W13 stage: k_gemm_xl<true> (256-row items) + k_gemm_large<true> (128-row "
                               "items) + k_w13_small<4> (items the exact-shape table sends to 16-row tiles) + "
                               "SwiGLU/requant",
                     "achieved": t13, "peak": MFMA_PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": t13 / MFMA_PEAK_FP8_TFLOPS, "frac_of_fp4_peak": t13 / MFMA_PEAK_FP4_TFLOPS,
                     "traffic": measured_traffic(w.name, ["moe::k_w13_small<4>", "moe::k_gemm_xl<true>",
                                                          "moe::k_gemm_large<true>"]),
                     "algorithmic_flops_per_launch": f13, "avg_launch_ms": p13_ms},
        "step_bounds": {"algorithmic_flops": flops, "algorithmic_bytes": step_bytes,
                        "mfma_frac": tstep / MFMA_PEAK_FP8_TFLOPS,
                        "hbm_frac": step_bytes / (ps * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "ideal_ms": max(flops / (MFMA_PEAK_FP8_TFLOPS * 1e9), step_bytes / (HBM_PEAK_GBS * 1e6))},
        "mall_flushed": {"ms_per_step": fl_step, "max_ms_per_step": fl_max, "value": w.T / (fl_step * 1e-3),
                         "w13_ms": fl_w13},
        "dense_fp8_gemm_reference": {
            "what": "hipBLASLt dense FP8 GEMM (torch._scaled_mm, per-tensor scales, bf16 out) on the dense "
                    "problem of each GEMM's total shape (all pairs as rows): context, not part of the step",
            "w13": ref13, "w2": ref2,
            "w13_stage_vs_reference": t13 / ref13["tflops"],
            "w2_stage_vs_reference": t2 / ref2["tflops"]},
        **({"shared_tflops": fs / (stages["shared"] * 1e-3) / 1e12} if w.Is else {}),
        "stage_ms_untimed_pass": stages,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=8)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["decode7", "decode7_chain", "decode7_a16", "decode7_nvfp4", "decode256",
                                       "decode256_a16", "decode256_nvfp4", "prefill32k", "tp8rank32k", "copy"],
                    default=None,
                    help="run one workload only (for profiling); prints its own JSON object. 'copy' runs "
                         "a 1 GiB device-to-device copy, the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # contents do not matter for a copy
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"workload": "copy", "bytes_read": src.numel(), "bytes_written": dst.numel(), "launches": 3}))
        return
    moe.lib()
    t = time.time()
    # one 384-expert set, shared by the full-size workloads, converted once to the
    # kernel-native layout (a weight-load step, outside every timed region)
    W_rows = make_expert_weights(WORKLOADS["decode7"], dev)   # row-major codes (the oracle's input)
    W = moe.pack_weights(W_rows)
    flush = torch.zeros(1 << 27, dtype=torch.int64, device=dev)    # 1 GiB, read to evict the cache
    torch.cuda.synchronize()
    log(f"[bench] weights generated and packed in {time.time() - t:.1f}s")

    if args.only is not None:
        chain = args.only == "decode7_chain"
        a16 = args.only.endswith("_a16")
        nv = args.only.endswith("_nvfp4")
        name = args.only.split("_")[0] if (chain or a16 or nv) else args.only
        if nv:
            r = Runner(name, dev, moe.pack_weights(make_expert_weights(WORKLOADS["decode7"], dev, fmt="nvfp4")),
                       flags=moe.FLAG_NVFP4)
        else:
            r = Runner(name, dev, W if args.only != "tp8rank32k" else None,
                       flags=moe.FLAG_DECODE_CHAIN if chain else (moe.FLAG_A16 if a16 else 0))
        if args.only.startswith("decode"):
            obj = decode_object(r, args.steps, args.warmup, flush)
        else:
            obj = prefill_object(r, args.prefill_steps, flush)
        print(json.dumps(obj))
        return

    # ---- decode verify, 7 tokens (headline)
    d7 = decode_object(Runner("decode7", dev, W), args.steps, args.warmup, flush)
    w = WORKLOADS["decode7"]
    out = {
        "metric": METRIC,
        "value": d7["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d7["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (E8M0 block scales), fp32 accumulate",
        "data": "synthetic (seeded: x N(0,1) bf16, Zipf routing, N(0,0.02) weights packed to MXFP4)",
        "config": d7["config"],
        "roofline": d7["roofline"],
        "step_hbm_gbs": d7["step_hbm_gbs"],
        "step_hbm_frac": d7["step_hbm_frac"],
        "mall_flushed": d7["mall_flushed"],
        "stage_ms_untimed_pass": d7["stage_ms_untimed_pass"],
    }
    # ---- the same verify as one persistent launch (MOE_FLAG_DECODE_CHAIN)
    out["decode7_chain"] = decode_object(Runner("decode7", dev, W, flags=moe.FLAG_DECODE_CHAIN), args.steps,
                                         args.warmup, flush)
    # ---- high-concurrency decode step, 256 tokens
    out["decode256"] = decode_object(Runner("decode256", dev, W), max(args.steps // 2, 5), args.warmup, flush)
    # ---- the same decode steps with bf16 activations (MXFP4A16, MOE_FLAG_A16)
    out["decode7_a16"] = decode_object(Runner("decode7", dev, W, flags=moe.FLAG_A16), args.steps, args.warmup, flush)
    out["decode256_a16"] = decode_object(Runner("decode256", dev, W, flags=moe.FLAG_A16), max(args.steps // 2, 5),
                                         args.warmup, flush)
    # ---- and with NVFP4 expert weights (the same float weights packed as NVFP4)
    W_nv = moe.pack_weights(make_expert_weights(WORKLOADS["decode7"], dev, fmt="nvfp4"))
    out["decode7_nvfp4"] = decode_object(Runner("decode7", dev, W_nv, flags=moe.FLAG_NVFP4), args.steps,
                                         args.warmup, flush)
    out["decode256_nvfp4"] = decode_object(Runner("decode256", dev, W_nv, flags=moe.FLAG_NVFP4),
                                           max(args.steps // 2, 5), args.warmup, flush)
    del W_nv

    # ---- prefill chunk, 32K tokens, and one MoE-TP8 rank of it
    if not args.no_prefill:
        out["prefill32k"] = prefill_object(Runner("prefill32k", dev, W), args.prefill_steps, flush)
        out["tp8rank32k"] = prefill_object(Runner("tp8rank32k", dev), args.prefill_steps, flush)

    # ---- oracle on the host cores (bounded samples)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline("decode7", W_rows, list(range(WORKLOADS["decode7"].T)))
        log(f"[bench] cpu_baseline {out['cpu_baseline']}")
        if not args.no_prefill:
            out["prefill32k"]["cpu_baseline"] = cpu_baseline("prefill32k", W_rows, list(range(32)))
            log(f"[bench] prefill32k cpu_baseline {out['prefill32k']['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
