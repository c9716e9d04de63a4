"""Workload table and seeded generators.

Shapes come from the DeepSeek-V4 MoE layer the sources serve: 384 routed experts
and top-8 routing ("Pushing the Limits of Serving DeepSeek-V4-Pro", §3.3), a
7-token target verify ("Optimization progress report", Optimization 06), a 32K
single prefill chunk (same blog, §3.2) and MoE-TP8 ranks (same blog, §3.1). The
hidden size 7168 and intermediate size 3072 per expert are the model's; one
MoE-TP8 rank owns 3072/8 = 384 intermediate columns.

Everything here is *input generation*: activations drawn N(0,1) and rounded to
bf16, router choices, and expert weights drawn N(0, 0.02) and packed into MXFP4
(E2M1 codes, one E8M0 scale per 32 along K) or, for the dense shared expert,
FP8 E4M3 codes with one E8M0 scale per 128x128 block. The packing uses the OCP
MX scale choice for *weights* (shared exponent = floor(log2(amax)) - emax of the
element type, saturating); the FFN never re-encodes weights, so none of this is
on its path.

Router-side streams (x, routing) use numpy's PCG64 and are identical on every
machine. Weights are drawn with ``torch.Generator`` on the device they are made
on (CPU for small workloads, the GPU for the 13.5 GB full-size set), one
generator per expert so any subset of experts can be regenerated alone.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size (K of W13, N of W2)
    I: int            # intermediate size per expert (per rank for a TP slice)
    E: int            # routed experts
    K: int            # top-k
    routing: str      # "softmax" | "zipf" | "affinity"
    seed: int         # base seed for x / routing streams
    zipf_s: float = 0.0
    Is: int = 0       # shared-expert intermediate size (0 = no shared expert)
    weight_seed: int = 90002
    # intermediate size of the full weight set this workload's weights are a
    # column slice of (rank 0 of an MoE-TP split); 0 = the weights are unsliced
    full_I: int = 0
    requests: int = 0        # affinity routing: number of requests
    subset: int = 0          # affinity routing: experts per request subset
    p_subset: float = 0.0    # affinity routing: probability a pick comes from the subset
    desc: str = ""

    @property
    def P(self) -> int:
        return self.T * self.K


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", T=64, H=256, I=512, E=8, K=2, routing="softmax", seed=1000,
                 weight_seed=10002,
                 desc="64 tokens, hidden 256, 8 experts, intermediate 512, top-2, softmax top-k"),
        Workload("decode7", T=7, H=7168, I=3072, E=384, K=8, routing="zipf", zipf_s=1.0,
                 seed=2000,
                 desc="7-token verify, 384 experts, Zipf s=1.0 routing"),
        Workload("decode256", T=256, H=7168, I=3072, E=384, K=8, routing="affinity",
                 zipf_s=1.1, seed=3000, requests=32, subset=16, p_subset=0.7,
                 desc="32 requests x 8 speculative positions, Zipf 1.1 + 70% per-request affinity"),
        Workload("prefill32k", T=32768, H=7168, I=3072, E=384, K=8, routing="zipf",
                 zipf_s=1.2, seed=4000,
                 desc="32K prefill chunk, Zipf s=1.2 routing"),
        Workload("tp8rank32k", T=32768, H=7168, I=384, E=384, K=8, routing="zipf",
                 zipf_s=1.2, seed=4000, Is=384, full_I=3072,
                 desc="one MoE-TP8 rank of the 32K prefill chunk + FP8 shared expert"),
    ]
}


def scaled(base: str, **over) -> Workload:
    """A copy of a workload with some fields replaced (used for small test shapes)."""
    return dataclasses.replace(WORKLOADS[base], **over)


# ----------------------------------------------------------------------------- routing

def _zipf_probs(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def make_routing(w: Workload):
    """Router output: (topk_ids int32 [T, K], topk_weights float32 [T, K]).

    * softmax: logits N(0,1) over E; top-k by logit (ties to the lower id); the
      weights are the softmax over the chosen logits (a renormalised top-k softmax).
    * zipf: expert of popularity rank r is drawn with p ~ r^-s, ranks mapped to
      experts by a seeded permutation; K distinct picks per token by Gumbel-top-k
      (successive sampling without replacement); weights = softmax of K N(0,1).
    * affinity: tokens come in requests of T/requests positions; each request owns
      a random subset of experts; every pick independently comes from the subset
      with probability p_subset, otherwise from the global Zipf law; a pick equal
      to an earlier pick of the same token is redrawn.
    """
    T, E, K = w.T, w.E, w.K
    rng = np.random.Generator(np.random.PCG64(w.seed + 1))
    if w.routing == "softmax":
        logits = rng.standard_normal((T, E))
        order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        chosen = np.take_along_axis(logits, order, axis=1)
        wts = _softmax(chosen)
        return order.astype(np.int32), wts.astype(np.float32)

    perm = np.random.Generator(np.random.PCG64(w.seed + 5)).permutation(E)
    p = _zipf_probs(E, w.zipf_s)
    if w.routing == "zipf":
        scores = np.log(p)[None, :] + rng.gumbel(size=(T, E))
        ranks = np.argsort(-scores, axis=1, kind="stable")[:, :K]
        ids = perm[ranks]
    elif w.routing == "affinity":
        arng = np.random.Generator(np.random.PCG64(w.seed + 5 + 1))
        per_req = T // w.requests
        assert per_req * w.requests == T
        ids = np.empty((T, K), dtype=np.int64)
        cdf = np.cumsum(p)
        for r in range(w.requests):
            subset = arng.choice(E, size=w.subset, replace=False)
            for t in range(r * per_req, (r + 1) * per_req):
                picked = []
                while len(picked) < K:
                    if arng.random() < w.p_subset:
                        e = int(subset[arng.integers(w.subset)])
                    else:
                        rank = int(np.searchsorted(cdf, arng.random() * cdf[-1], side="right"))
                        e = int(perm[min(rank, E - 1)])
                    if e not in picked:
                        picked.append(e)
                ids[t] = picked
    else:
        raise ValueError(w.routing)
    wts = _softmax(rng.standard_normal((T, K)))
    return ids.astype(np.int32), wts.astype(np.float32)


def make_x(w: Workload) -> torch.Tensor:
    """Token activations: N(0,1) float32 rounded to bf16 (CPU tensor [T, H])."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 0))
    x = rng.standard_normal((w.T, w.H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


# ----------------------------------------------------------------------------- weights

def _e2m1_pack(v: torch.Tensor, N: int, Kd: int) -> torch.Tensor:
    """Elements already divided by their scales -> E2M1 codes rounded to
    nearest-even on the grid and saturated at +-6, two per byte (low nibble = even k)."""
    a = v.abs()
    q = torch.where(a < 2, 0.5, torch.where(a < 4, 1.0, 2.0))
    r = torch.clamp(torch.round(a / q) * q, max=6.0)
    idx = torch.where(r < 2, r * 2, torch.where(r < 4, r + 2, r / 2 + 4)).to(torch.uint8)
    code = idx | (torch.signbit(v).to(torch.uint8) << 3)
    code = code.reshape(N, Kd)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()


def _pack_mxfp4(wf: torch.Tensor):
    """Pack float weights [N, K] into MXFP4: codes [N, K/2] u8 (low nibble = even k)
    and E8M0 scales [N, K/32] u8, with the OCP MX weight rule (shared exponent
    floor(log2 amax) - 2, elements rounded to nearest-even on the E2M1 grid and
    saturated at +-6)."""
    N, Kd = wf.shape
    blk = wf.reshape(N, Kd // 32, 32)
    amax = blk.abs().amax(-1)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    X = torch.where(amax > 0, ex - 3, torch.full_like(ex, -127)).clamp(-127, 127)
    v = blk * torch.exp2(-X.to(torch.float32)).unsqueeze(-1)
    return _e2m1_pack(v, N, Kd), (X + 127).to(torch.uint8).contiguous()


def _pack_nvfp4(wf: torch.Tensor):
    """Pack one float weight tensor [N, K] into NVFP4 (NVIDIA's published recipe):
    a tensor scale gs = amax / (6 * 448) (float32), one E4M3 scale per 16 elements
    s = E4M3(block amax / (6 gs)) (nearest), elements rounded to nearest-even on the
    E2M1 grid of w / (s gs) and saturated at +-6. Returns codes [N, K/2] u8, block
    scales [N, K/16] u8 (E4M3 bits) and gs."""
    N, Kd = wf.shape
    gs = (wf.abs().amax() / (6.0 * 448.0)).clamp(min=2.0 ** -100).to(torch.float32)
    blk = wf.reshape(N, Kd // 16, 16)
    s8 = (blk.abs().amax(-1) / (6.0 * gs)).clamp(max=448.0).to(torch.float8_e4m3fn)
    sv = s8.to(torch.float32) * gs
    v = torch.where(sv.unsqueeze(-1) > 0, blk / sv.unsqueeze(-1), torch.zeros_like(blk))
    return _e2m1_pack(v, N, Kd), s8.view(torch.uint8).contiguous(), float(gs)


def _pack_fp8_block(wf: torch.Tensor):
    """Pack float weights [N, K] into FP8 E4M3 codes [N, K] with one E8M0 scale per
    128x128 block ([N/128, K/128]); OCP MX weight rule, saturating at 448."""
    N, Kd = wf.shape
    blk = wf.reshape(N // 128, 128, Kd // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    _, ex = torch.frexp(amax)
    X = torch.where(amax > 0, ex - 9, torch.full_like(ex, -127)).clamp(-127, 127)
    v = blk * torch.exp2(-X.to(torch.float32))[:, None, :, None]
    codes = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.reshape(N, Kd).contiguous(), (X + 127).to(torch.uint8).contiguous()


def _gen_device(w: Workload, device) -> torch.device:
    dev = torch.device(device)
    # small weight sets are drawn on the CPU so CPU and GPU runs see the same bytes
    n = w.E * (2 * (w.full_I or w.I) * w.H + w.H * (w.full_I or w.I))
    return torch.device("cpu") if n <= (1 << 27) else dev


def make_expert_weights(w: Workload, device="cpu", experts: Optional[Sequence[int]] = None, fmt: str = "mxfp4"):
    """4-bit expert weights on ``device``.

    Returns dict with w13 [E, 2I, H/2], w13_s [E, 2I, H/32], w2 [E, H, I/2],
    w2_s [E, H, I/32] (all uint8). W13 rows [0, I) are the gate projection and
    rows [I, 2I) the up projection. ``experts`` restricts generation to a subset
    (the returned tensors then have len(experts) rows in that order).
    fmt="nvfp4": the same float weights packed as NVFP4: w13_s [E, 2I, H/16] and
    w2_s [E, H, I/16] E4M3 block scales, plus w13_gs / w2_gs [E] float32 tensor
    scales (one per expert and projection).
    """
    if fmt not in ("mxfp4", "nvfp4"):
        raise ValueError(fmt)
    nv = fmt == "nvfp4"
    blk = 16 if nv else 32
    dev = torch.device(device)
    gdev = _gen_device(w, dev)
    ex = list(range(w.E)) if experts is None else list(experts)
    fI = w.full_I or w.I
    H, I = w.H, w.I
    w13 = torch.empty((len(ex), 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13_s = torch.empty((len(ex), 2 * I, H // blk), dtype=torch.uint8, device=dev)
    w2 = torch.empty((len(ex), H, I // 2), dtype=torch.uint8, device=dev)
    w2_s = torch.empty((len(ex), H, I // blk), dtype=torch.uint8, device=dev)
    gs13 = torch.empty(len(ex), dtype=torch.float32)
    gs2 = torch.empty(len(ex), dtype=torch.float32)
    g = torch.Generator(device=gdev)
    for i, e in enumerate(ex):
        g.manual_seed(w.weight_seed * 4096 + e)
        f13 = torch.randn((2 * fI, H), generator=g, device=gdev, dtype=torch.float32) * 0.02
        if fI != I:   # rank-0 column slice of the full gate and up projections
            f13 = torch.cat([f13[:I], f13[fI:fI + I]], 0)
        if nv:
            c, s, gs13[i] = _pack_nvfp4(f13)
        else:
            c, s = _pack_mxfp4(f13)
        w13[i].copy_(c)
        w13_s[i].copy_(s)
        del f13
        g.manual_seed((w.weight_seed + 1) * 4096 + e)
        f2 = torch.randn((H, fI), generator=g, device=gdev, dtype=torch.float32) * 0.02
        if fI != I:
            f2 = f2[:, :I].contiguous()
        if nv:
            c, s, gs2[i] = _pack_nvfp4(f2)
        else:
            c, s = _pack_mxfp4(f2)
        w2[i].copy_(c)
        w2_s[i].copy_(s)
        del f2
    out = {"w13": w13, "w13_s": w13_s, "w2": w2, "w2_s": w2_s}
    if nv:
        out.update(w13_gs=gs13.to(dev), w2_gs=gs2.to(dev))
    return out


def make_shared_weights(w: Workload, device="cpu"):
    """Dense shared expert with FP8 E4M3 weights and 128x128 E8M0 block scales:
    w13s [2Is, H], w13s_s [2Is/128, H/128], w2s [H, Is], w2s_s [H/128, Is/128]."""
    if not w.Is:
        return None
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 4)
    f13 = torch.randn((2 * w.Is, w.H), generator=g, device=dev) * 0.02
    f2 = torch.randn((w.H, w.Is), generator=g, device=dev) * 0.02
    c13, s13 = _pack_fp8_block(f13)
    c2, s2 = _pack_fp8_block(f2)
    return {"w13s": c13, "w13s_s": s13, "w2s": c2, "w2s_s": s2}


def slice_experts(weights: dict, experts: Sequence[int], device="cpu") -> dict:
    """Copy the packed weights of a subset of experts (in the given order) to ``device``."""
    idx = torch.as_tensor(list(experts), dtype=torch.long, device=weights["w13"].device)
    return {k: v.index_select(0, idx).to(device) for k, v in weights.items()}


@dataclasses.dataclass
class MoEInputs:
    wl: Workload
    x: torch.Tensor              # bf16 [T, H]
    topk_ids: torch.Tensor       # int32 [T, K]
    topk_weights: torch.Tensor   # float32 [T, K]
    weights: Optional[dict]      # MXFP4 expert weights (see make_expert_weights)
    shared: Optional[dict]       # FP8 shared expert (see make_shared_weights) or None

    def to(self, device) -> "MoEInputs":
        mv = lambda d: None if d is None else {k: v.to(device) for k, v in d.items()}
        return MoEInputs(self.wl, self.x.to(device), self.topk_ids.to(device),
                         self.topk_weights.to(device), mv(self.weights), mv(self.shared))


def make_inputs(wl, device="cpu", weights: bool = True) -> MoEInputs:
    """All inputs of one workload (by name or Workload) on ``device``."""
    w = WORKLOADS[wl] if isinstance(wl, str) else wl
    ids, wts = make_routing(w)
    x = make_x(w).to(device)
    W = make_expert_weights(w, device) if weights else None
    S = make_shared_weights(w, device) if (weights and w.Is) else None
    return MoEInputs(w, x, torch.from_numpy(ids).to(device), torch.from_numpy(wts).to(device), W, S)


def routing_stats(ids: np.ndarray, E: int) -> dict:
    """Per-expert pair counts of a routing (used for reporting and tests)."""
    c = np.bincount(ids.ravel(), minlength=E)
    nz = c[c > 0]
    return {"distinct": int((c > 0).sum()), "max": int(c.max()), "median_nonzero": float(np.median(nz)) if nz.size else 0.0,
            "counts": c}


__all__ = ["Workload", "WORKLOADS", "scaled", "make_routing", "make_x", "make_expert_weights",
           "make_shared_weights", "slice_experts", "MoEInputs", "make_inputs", "routing_stats"]
