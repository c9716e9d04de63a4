"""moe_ffn_static (the entry point that allocates nothing, for callers that
cannot call hipMalloc) against moe_ffn on the same inputs, through the C-ABI:
bit-identical y and SwiGLU codes on two calls in a row on one GPU (the second
smaller, so it runs over the first call's leftovers in the static scratch), with
and without the shared expert, and with bf16 activations (MOE_FLAG_A16), also with
every intermediate row (activation codes, SwiGLU rows, per-pair rows) held in the
static scratch; a call whose workspace exceeds the static scratch is refused on
the host with MOE_ESCRATCH and leaves y untouched."""

import numpy as np
import pytest
import torch

import mxfp4_weights_fp8_amd as moe
from gpu_helpers import say
from synth import make_inputs, scaled

pytestmark = pytest.mark.gpu


def _both(inp):
    w = inp.wl
    p = moe.plan(inp.topk_ids, w.E, w.H, w.I, Is=w.Is if inp.shared else 0)
    W = moe.pack_weights(inp.weights)
    y_ws, dbg_ws = moe.ffn(inp.x, inp.topk_weights, p, W, shared=inp.shared, debug=True)
    y_st, dbg_st = moe.ffn(inp.x, inp.topk_weights, p, W, shared=inp.shared, debug=True, static=True)
    torch.cuda.synchronize()
    return (y_ws, dbg_ws), (y_st, dbg_st)


@pytest.mark.parametrize("shared", [False, True])
def test_static_scratch_matches_workspace_on_consecutive_calls(gpu, shared):
    big = scaled("tiny", T=300, H=1024, I=512, E=6, K=4, Is=256 if shared else 0, seed=71, weight_seed=71,
                 name="static_big")
    small = scaled("tiny", T=5, H=1024, I=512, E=6, K=4, Is=256 if shared else 0, seed=72, weight_seed=72,
                   name="static_small")
    for wl in (big, small):
        inp = make_inputs(wl).to(gpu)
        d = moe.make_dims(wl.T, wl.H, wl.I, wl.E, wl.K, wl.Is if shared else 0)
        assert moe.ffn_workspace_bytes(d) <= moe.FFN_STATIC_MAX_BYTES
        (y0, g0), (y1, g1) = _both(inp)
        say(f"[static scratch] T={wl.T} shared={shared} ws={moe.ffn_workspace_bytes(d)} B")
        assert torch.equal(y0, y1)
        for k in ("x_q", "x_s", "h_q", "h_s") + (("sh_q", "sh_s") if shared else ()):
            assert torch.equal(g0[k], g1[k]), k


@pytest.mark.parametrize("flags", [0, moe.FLAG_A16])
def test_static_scratch_holds_every_intermediate(gpu, flags):
    """No debug outputs: the activation codes, SwiGLU rows and per-pair rows all
    live in the scratch; y bit-identical to moe_ffn's on two calls in a row."""
    for T, seed in ((300, 74), (5, 75)):
        wl = scaled("tiny", T=T, H=1024, I=512, E=6, K=4, seed=seed, weight_seed=seed, name="static_nodbg")
        inp = make_inputs(wl).to(gpu)
        p = moe.plan(inp.topk_ids, wl.E, wl.H, wl.I, flags=flags)
        assert moe.ffn_workspace_bytes(p.dims) <= moe.FFN_STATIC_MAX_BYTES
        W = moe.pack_weights(inp.weights)
        y_ws = moe.ffn(inp.x, inp.topk_weights, p, W)
        y_st = moe.ffn(inp.x, inp.topk_weights, p, W, static=True)
        torch.cuda.synchronize()
        say(f"[static scratch, no debug] T={T} flags={flags}")
        assert torch.equal(y_ws, y_st)


def test_static_scratch_refuses_oversized_calls(gpu):
    wl = scaled("tiny", T=4096, H=1024, I=512, E=6, K=8, seed=73, weight_seed=73, name="static_over")
    d = moe.make_dims(wl.T, wl.H, wl.I, wl.E, wl.K)
    assert moe.ffn_workspace_bytes(d) > moe.FFN_STATIC_MAX_BYTES
    inp = make_inputs(wl).to(gpu)
    p = moe.plan(inp.topk_ids, wl.E, wl.H, wl.I)
    W = moe.pack_weights(inp.weights)
    y = torch.full((wl.T, wl.H), 7.0, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(moe.MoEError) as e:
        moe.ffn(inp.x, inp.topk_weights, p, W, y=y, static=True)
    assert e.value.code == moe.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
