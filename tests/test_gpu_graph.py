"""Graph replay of a whole step (GB10 report, Optimization 13: the decode step is
captured once and replayed). moe_plan + moe_ffn only enqueue kernels (no host
synchronization, no allocation, no memset), so both can be captured into one HIP
graph. Each replay reads new routing and activations that were written into the
captured input buffers, with eager work and synchronizations between replays, and
must give bit for bit the plan and the output of an eager run on the same inputs.
Two independent steps enqueued on two streams at once must match their sequential
runs (the calls keep no state of their own)."""

import pytest
import torch

import mxfp4_weights_fp8_amd as moe
from gpu_helpers import say
from synth import make_expert_weights, make_inputs, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev(gpu):
    moe.lib()
    return gpu


@pytest.mark.parametrize("T,H,I,E,K,Is,flags", [
    (300, 512, 512, 3, 2, 0, 0),      # 256-row and 128-row large-M items
    (7, 256, 256, 64, 8, 128, 0),     # decode-sized: small-M tiles only, plus the dense shared expert
    (400, 1280, 384, 2, 1, 0, 0),     # W2 with three K steps (few-K kernel)
    (600, 256, 256, 16, 4, 0, 0),     # 2400 pairs: the four-launch plan
    (300, 512, 512, 3, 2, 0, moe.FLAG_A16),           # bf16 activations
    (7, 256, 256, 64, 8, 0, moe.FLAG_DECODE_CHAIN),   # the persistent chain (counters zeroed by a kernel)
    (300, 512, 512, 3, 2, 0, moe.FLAG_NVFP4),         # NVFP4 weights
])
def test_graph_replay_matches_eager(dev, T, H, I, E, K, Is, flags):
    base = scaled("tiny", T=T, H=H, I=I, E=E, K=K, Is=Is, seed=70, weight_seed=71, name="graph")
    first = make_inputs(base).to(dev)
    if flags & moe.FLAG_NVFP4:
        first.weights = make_expert_weights(base, dev, fmt="nvfp4")
    W = moe.pack_weights(first.weights)
    shared = first.shared
    ids, x, tw = first.topk_ids.clone(), first.x.clone(), first.topk_weights.clone()

    # buffers the graph captures (allocated, and the path run once, before capture)
    pbuf = moe.plan(ids, E, H, I, Is=Is, flags=flags)
    ws = torch.empty(moe.ffn_workspace_bytes(pbuf.dims), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.plan(ids, E, H, I, Is=Is, flags=flags, out=pbuf)
        moe.ffn(x, tw, pbuf, W, shared=shared, ws=ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.plan(ids, E, H, I, Is=Is, flags=flags, out=pbuf)
        moe.ffn(x, tw, pbuf, W, shared=shared, ws=ws, y=y)
    torch.cuda.synchronize()

    for rep in range(3):
        nxt = make_inputs(scaled("tiny", T=T, H=H, I=I, E=E, K=K, Is=Is, seed=80 + rep, weight_seed=71,
                                 name="graph"), weights=False).to(dev)
        ids.copy_(nxt.topk_ids)
        x.copy_(nxt.x)
        tw.copy_(nxt.topk_weights)
        g.replay()
        torch.cuda.synchronize()
        y_graph = y.clone()
        pairs_graph = pbuf.sorted_pairs.clone()
        offsets_graph = pbuf.expert_offsets.clone()
        # eager run on the same inputs, fresh buffers
        p2 = moe.plan(ids, E, H, I, Is=Is, flags=flags)
        y2 = moe.ffn(x, tw, p2, W, shared=shared)
        torch.cuda.synchronize()
        assert torch.equal(offsets_graph, p2.expert_offsets), f"replay {rep}: expert offsets differ"
        assert torch.equal(pairs_graph, p2.sorted_pairs), f"replay {rep}: plan differs"
        assert torch.equal(y_graph.view(torch.int16), y2.view(torch.int16)), f"replay {rep}: y differs"
        assert bool(torch.isfinite(y2.float()).all())
        say(f"[graph {T}x{H} I{I} E{E} K{K} Is{Is} flags{flags}] replay {rep} equal to eager")


def test_two_streams_match_sequential(dev):
    """Two independent steps (different shapes, weights and routing) enqueued on two
    streams before either is synchronized give bit for bit the outputs of running
    them one after the other: the library keeps no state between calls."""
    cases = []
    for T, H, I, E, K, seed in [(300, 512, 512, 3, 2, 90), (7, 256, 384, 16, 8, 91)]:
        wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"st{seed}")
        inp = make_inputs(wl).to(dev)
        W = moe.pack_weights(inp.weights)
        p = moe.plan(inp.topk_ids, E, H, I)
        y = moe.ffn(inp.x, inp.topk_weights, p, W)
        torch.cuda.synchronize()
        cases.append((inp, W, y.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for (inp, W, _), s in zip(cases, streams):
        with torch.cuda.stream(s):
            w = inp.wl
            p = moe.plan(inp.topk_ids, w.E, w.H, w.I)
            outs.append(moe.ffn(inp.x, inp.topk_weights, p, W))
    torch.cuda.synchronize()
    for (inp, _, y_seq), y in zip(cases, outs):
        assert torch.equal(y.view(torch.int16), y_seq.view(torch.int16)), f"{inp.wl.name}: concurrent != sequential"
