"""GPU parity of the bf16-activation variant (MXFP4A16, moe_dims.flags =
MOE_FLAG_A16): the HIP path through the C-ABI against the oracle's act="bf16"
mode. y within max-rel 2e-2 / mean-rel 2e-3; every bf16 SwiGLU output equal to
the oracle's or, where it differs, the bf16 rounding of a value inside the
hardware-dot envelope (tests/gpu_helpers.py)."""

import numpy as np
import pytest
import torch

import mxfp4_weights_fp8_amd as moe
from gpu_helpers import check_ffn_a16, check_plan, run_path, say, u16
from synth import WORKLOADS, make_expert_weights, make_inputs, scaled

pytestmark = pytest.mark.gpu

A16 = moe.FLAG_A16


@pytest.fixture(scope="module")
def dev(gpu):
    moe.lib()
    return gpu


@pytest.mark.parametrize("T,H,I,E,K,seed", [
    (1, 128, 128, 1, 1, 71),       # degenerate: one token, one expert, one K step
    (64, 256, 512, 8, 2, 72),      # the tiny workload's shape
    (33, 384, 384, 5, 3, 73),      # 3 K steps (no 4-step ring), ragged 16-row tiles
    (17, 1280, 1152, 40, 8, 74),   # 10 and 9 K steps, many experts
    (300, 512, 512, 1, 1, 75),     # one expert with a 256-row item and a remainder
    (700, 256, 768, 2, 1, 76),     # 256-row items of two experts
    (400, 1024, 256, 3, 2, 77),    # 128-row items
    (3, 16384, 256, 4, 2, 78),     # H at the small-M limit (scale runs of 8 KB per wave)
    (2, 256, 16384, 2, 1, 79),     # I at the small-M limit
    (30, 512, 256, 48, 16, 82),    # top-16: two batches of 8 picks in the combine
])
def test_a16_shapes(dev, T, H, I, E, K, seed):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"a16_{seed}")
    inp = make_inputs(wl).to(dev)
    p, (y, dbg) = run_path(inp, flags=A16)
    check_plan(p, inp.topk_ids.cpu().numpy(), E)
    check_ffn_a16(inp, p, y, dbg, label=f"{T}x{H} I{I} E{E} K{K}")


def test_a16_dropped_ids(dev):
    inp = make_inputs("tiny").to(dev)
    ids = inp.topk_ids.clone()
    ids[::5, 1] = -3
    ids[3, 0] = 99
    inp.topk_ids = ids
    p, (y, dbg) = run_path(inp, flags=A16)
    assert int(p.status.cpu()[0]) == int((ids < 0).sum() + (ids >= inp.wl.E).sum())
    check_ffn_a16(inp, p, y, dbg, label="tiny with dropped ids")


def test_a16_all_dropped_and_empty(dev):
    """Every pick dropped: y = 0. T = 0: a valid no-op."""
    inp = make_inputs(scaled("tiny", T=9, name="a16drop")).to(dev)
    inp.topk_ids = torch.full_like(inp.topk_ids, -1)
    _, (y, _) = run_path(inp, flags=A16)
    assert not u16(y).any()
    wl = scaled("tiny", T=1, name="a16empty")
    W = moe.pack_weights(make_inputs(wl).to(dev).weights)
    p = moe.plan(torch.zeros((0, wl.K), dtype=torch.int32, device=dev), wl.E, wl.H, wl.I, flags=A16)
    y = moe.ffn(torch.zeros((0, wl.H), dtype=torch.bfloat16, device=dev),
                torch.zeros((0, wl.K), dtype=torch.float32, device=dev), p, W)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, wl.H)


def test_a16_repeatable_and_chain_flag_ignored(dev):
    """Bitwise the same on a second call with a workspace full of other bytes, and
    with MOE_FLAG_DECODE_CHAIN added (which the variant ignores)."""
    inp = make_inputs(scaled("tiny", T=40, H=1024, I=512, E=16, K=4, seed=80, weight_seed=80, name="a16rep")).to(dev)
    packed = moe.pack_weights(inp.weights)
    outs = []
    for flags, fill in ((A16, 0x00), (A16, 0x7B), (A16 | moe.FLAG_DECODE_CHAIN, 0xFF)):
        p = moe.plan(inp.topk_ids, inp.wl.E, inp.wl.H, inp.wl.I, flags=flags)
        ws = torch.full((moe.ffn_workspace_bytes(p.dims),), fill, dtype=torch.uint8, device=dev)
        y = moe.ffn(inp.x, inp.topk_weights, p, packed, ws=ws)
        torch.cuda.synchronize()
        outs.append(u16(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_a16_is_not_the_fp8_path(dev):
    """The flag changes the computation: the FP8 path's y differs from the
    variant's by the activation quantization."""
    inp = make_inputs(scaled("tiny", T=16, seed=81, weight_seed=81, name="a16vs8")).to(dev)
    _, y16 = run_path(inp, flags=A16, debug=False)
    _, y8 = run_path(inp, debug=False)
    a, b = u16(y16), u16(y8)
    assert not np.array_equal(a, b)


@pytest.fixture(scope="module")
def full_weights(dev):
    """The 384-expert MXFP4 weight set of the H 7168 / I 3072 workloads."""
    import time
    t = time.time()
    W = make_expert_weights(WORKLOADS["decode7"], dev)
    torch.cuda.synchronize()
    say(f"[full weights] generated in {time.time() - t:.1f}s")
    return W


def _full_inputs(name, dev, W):
    inp = make_inputs(name, weights=False).to(dev)
    inp.weights = W
    return inp


def test_a16_decode7_full(dev, full_weights):
    """7-token verify at full size (H 7168, I 3072, 384 experts, top-8), every
    token and pick."""
    inp = _full_inputs("decode7", dev, full_weights)
    p, (y, dbg) = run_path(inp, flags=A16)
    check_ffn_a16(inp, p, y, dbg, label="decode7 full")


@pytest.mark.timeout(600)
def test_a16_decode256_full(dev, full_weights):
    """32 requests x 8 speculative positions at full size, every token and pick."""
    inp = _full_inputs("decode256", dev, full_weights)
    p, (y, dbg) = run_path(inp, flags=A16)
    check_ffn_a16(inp, p, y, dbg, label="decode256 full")
