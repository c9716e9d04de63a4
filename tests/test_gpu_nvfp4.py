"""GPU parity of NVFP4 expert weights (moe_ffn_nvfp4, moe_dims.flags =
MOE_FLAG_NVFP4): E2M1 codes, one E4M3 scale per 16 elements and one fp32 scale per
expert tensor, bf16 activations, against the oracle's ffn_ref_nvfp4. y within
max-rel 2e-2 / mean-rel 2e-3; every bf16 SwiGLU output equal to the oracle's or
the bf16 rounding of a value inside the hardware-dot envelope."""

import numpy as np
import pytest
import torch

import mxfp4_weights_fp8_amd as moe
from gpu_helpers import check_ffn_a16, check_plan, say, u16
from synth import WORKLOADS, make_expert_weights, make_inputs, scaled

pytestmark = pytest.mark.gpu

NV = moe.FLAG_NVFP4


@pytest.fixture(scope="module")
def dev(gpu):
    moe.lib()
    return gpu


def _run(inp, flags=NV, debug=True, ws=None):
    w = inp.wl
    p = moe.plan(inp.topk_ids, w.E, w.H, w.I, flags=flags)
    packed = moe.pack_weights(inp.weights)
    out = moe.ffn(inp.x, inp.topk_weights, p, packed, debug=debug, ws=ws)
    torch.cuda.synchronize()
    return p, out


def _inputs(wl, dev):
    inp = make_inputs(wl, weights=False).to(dev)
    inp.weights = make_expert_weights(wl, dev, fmt="nvfp4")
    return inp


@pytest.mark.parametrize("T,H,I,E,K,seed", [
    (1, 128, 128, 1, 1, 101),      # degenerate: one token, one expert, one K step
    (64, 256, 512, 8, 2, 102),     # the tiny workload's shape
    (33, 384, 384, 5, 3, 103),     # 3 K steps (no 4-step ring), ragged 16-row tiles
    (17, 1280, 1152, 40, 8, 104),  # 10 and 9 K steps, many experts
    (300, 512, 512, 1, 1, 105),    # a 256-row item and a remainder
    (400, 1024, 256, 3, 2, 106),   # 128-row items
    (700, 384, 384, 3, 1, 107),    # above 512 pairs (the wider work split), H of three 128-column blocks
    (20, 256, 256, 40, 12, 108),   # top-12: a partial second batch of picks in the combine
])
def test_nvfp4_shapes(dev, T, H, I, E, K, seed):
    inp = _inputs(scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"nv_{seed}"), dev)
    p, (y, dbg) = _run(inp)
    check_plan(p, inp.topk_ids.cpu().numpy(), E)
    check_ffn_a16(inp, p, y, dbg, label=f"{T}x{H} I{I} E{E} K{K}", nvfp4=True)


def test_nvfp4_dropped_ids_and_scale_edge_cases(dev):
    """Dropped picks; a zero block scale and subnormal E4M3 block scales in the
    weights of the experts in use."""
    inp = _inputs(scaled("tiny", T=40, seed=107, weight_seed=107, name="nvedge"), dev)
    ids = inp.topk_ids.clone()
    ids[::5, 1] = -3
    inp.topk_ids = ids
    W = inp.weights
    W["w13_s"][:, 0, :4] = 0            # gate row 0: first 64 K zero
    W["w13_s"][:, 1, 2] = 0x01          # smallest subnormal scale
    W["w13_s"][:, 2, :] = 0x05          # subnormal scales on a whole row
    W["w2_s"][:, 3, 1] = 0
    p, (y, dbg) = _run(inp)
    check_ffn_a16(inp, p, y, dbg, label="edge scales, dropped ids", nvfp4=True)


def test_nvfp4_entry_point_checks(dev):
    """moe_ffn refuses NVFP4 dims (it takes no tensor scales); the NVFP4 path needs
    the flag; the result does not depend on the workspace's prior contents."""
    inp = _inputs(scaled("tiny", T=20, H=512, I=256, E=6, K=2, seed=108, weight_seed=108, name="nvchk"), dev)
    packed = moe.pack_weights(inp.weights)
    w = inp.wl
    p = moe.plan(inp.topk_ids, w.E, w.H, w.I, flags=NV)
    outs = []
    for fill in (0x00, 0xA5):
        ws = torch.full((moe.ffn_workspace_bytes(p.dims),), fill, dtype=torch.uint8, device=dev)
        outs.append(u16(moe.ffn(inp.x, inp.topk_weights, p, packed, ws=ws)))
    assert np.array_equal(outs[0], outs[1])
    import ctypes
    d = p.dims
    ws = torch.empty(moe.ffn_workspace_bytes(d), dtype=torch.uint8, device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = moe.lib().moe_ffn(ctypes.byref(d), ptr(inp.x), ptr(inp.topk_weights), ptr(p.expert_offsets),
                           ptr(p.sorted_pairs), ptr(p.pair_rows), ptr(p.ws), ptr(packed["w13"]), ptr(packed["w13_s"]),
                           ptr(packed["w2"]), ptr(packed["w2_s"]), None, ptr(y), None, ptr(ws), ws.numel(), st)
    assert rc == moe.MOE_EINVAL
    d0 = moe.make_dims(w.T, w.H, w.I, w.E, w.K)
    rc = moe.lib().moe_ffn_nvfp4(ctypes.byref(d0), ptr(inp.x), ptr(inp.topk_weights), ptr(p.expert_offsets),
                                 ptr(p.sorted_pairs), ptr(p.pair_rows), ptr(p.ws), ptr(packed["w13"]),
                                 ptr(packed["w13_s"]), ptr(packed["w13_gs"]), ptr(packed["w2"]), ptr(packed["w2_s"]),
                                 ptr(packed["w2_gs"]), ptr(y), None, ptr(ws), ws.numel(), st)
    assert rc == moe.MOE_EINVAL
    rc = moe.lib().moe_ffn_nvfp4(ctypes.byref(d), ptr(inp.x), ptr(inp.topk_weights), ptr(p.expert_offsets),
                                 ptr(p.sorted_pairs), ptr(p.pair_rows), ptr(p.ws), ptr(packed["w13"]),
                                 ptr(packed["w13_s"]), None, ptr(packed["w2"]), ptr(packed["w2_s"]),
                                 ptr(packed["w2_gs"]), ptr(y), None, ptr(ws), ws.numel(), st)
    assert rc == moe.MOE_EINVAL
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def full_weights(dev):
    """The 384-expert set of the H 7168 / I 3072 workloads, packed as NVFP4."""
    import time
    t = time.time()
    W = make_expert_weights(WORKLOADS["decode7"], dev, fmt="nvfp4")
    torch.cuda.synchronize()
    say(f"[full nvfp4 weights] generated in {time.time() - t:.1f}s")
    return W


def _full_inputs(name, dev, W):
    inp = make_inputs(name, weights=False).to(dev)
    inp.weights = W
    return inp


def test_nvfp4_decode7_full(dev, full_weights):
    inp = _full_inputs("decode7", dev, full_weights)
    p, (y, dbg) = _run(inp)
    check_ffn_a16(inp, p, y, dbg, label="decode7 full", nvfp4=True)


@pytest.mark.timeout(600)
def test_nvfp4_decode256_full(dev, full_weights):
    inp = _full_inputs("decode256", dev, full_weights)
    p, (y, dbg) = _run(inp)
    check_ffn_a16(inp, p, y, dbg, label="decode256 full", nvfp4=True)
