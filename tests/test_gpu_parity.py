"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the same
seeded inputs. Plans and activation codes bit-exact; SwiGLU codes: at most 0.1%
differ, by one grid step, except a capped count that must round from inside the
hardware-dot envelope (tests/gpu_helpers.py); y within max-rel 2e-2 / mean-rel
2e-3. The full-size workloads are compared on every token and every pair."""

import numpy as np
import pytest
import torch

import mxfp4_weights_fp8_amd as moe
from gpu_helpers import MAX_REL, check_ffn, check_plan, run_path, say, u16
from oracle.formats import bf16_to_f64
from oracle.moe import ffn_ref, plan_ref, quant_act_ref
from synth import WORKLOADS, make_expert_weights, make_inputs, make_routing, make_shared_weights, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev(gpu):
    moe.lib()
    return gpu


# ----------------------------------------------------------------------------- weight layout

def test_pack_weights_layout(dev):
    """moe_pack_weights against the layout definition written out in numpy: block
    (g, s) of 16 rows x 128 K at g*16*(K/2) + s*1024, byte 16*(16q + c) + b =
    w[16g + c][64s + 16q + b]; bit-exact, both tensors, and the scales untouched."""
    g = torch.Generator().manual_seed(7)
    E, H, I = 3, 384, 256
    W = {"w13": torch.randint(0, 256, (E, 2 * I, H // 2), generator=g, dtype=torch.uint8),
         "w13_s": torch.randint(0, 256, (E, 2 * I, H // 32), generator=g, dtype=torch.uint8),
         "w2": torch.randint(0, 256, (E, H, I // 2), generator=g, dtype=torch.uint8),
         "w2_s": torch.randint(0, 256, (E, H, I // 32), generator=g, dtype=torch.uint8)}
    packed = moe.pack_weights({k: v.to(dev) for k, v in W.items()})
    torch.cuda.synchronize()

    def expect(w):
        R, kb = w.shape[0] * w.shape[1], w.shape[2]
        a = w.numpy().reshape(R // 16, 16, kb // 64, 4, 16)      # [g, c, s, q, b]
        return a.transpose(0, 2, 3, 1, 4).reshape(w.shape)      # [g, s, q, c, b]

    for k in ("w13", "w2"):
        assert np.array_equal(packed[k].cpu().numpy(), expect(W[k])), k
    for k in ("w13_s", "w2_s"):
        assert np.array_equal(packed[k].cpu().numpy(), W[k].numpy()), k
    assert packed["layout"] == "packed"
    with pytest.raises(ValueError):
        moe.ffn(torch.zeros((1, H), dtype=torch.bfloat16, device=dev), torch.ones((1, 1), device=dev),
                moe.plan(torch.zeros((1, 1), dtype=torch.int32, device=dev), E, H, I), {k: v.to(dev) for k, v in W.items()})


# ----------------------------------------------------------------------------- quantizer

def test_quant_act_every_bf16_value(dev):
    """Every finite bf16 pattern, shuffled into 128-column blocks (so block scales
    span the whole exponent range), plus zero blocks and blocks whose amax sits on
    and next to a scale boundary 1.75 * 2^p: codes and scales bit-exact."""
    allv = np.arange(65536, dtype=np.uint16)
    fin = allv[np.isfinite(bf16_to_f64(allv))]
    rows = []
    for seed in range(3):
        perm = np.random.default_rng(seed).permutation(fin)
        n = perm.size // 128 * 128
        rows.append(perm[:n].reshape(-1, 128))
    sorted_rows = np.sort(fin)[: fin.size // 128 * 128].reshape(-1, 128)   # narrow-range blocks
    rows.append(sorted_rows)
    special = np.zeros((8, 128), dtype=np.uint16)                          # zeros, -0, boundaries
    special[1, :] = 0x8000
    b175 = np.float32(1.75).view(np.uint32) >> 16                          # bf16 1.75
    special[2, 0] = b175
    special[3, 0] = b175 + 1
    special[4, 5] = b175 | 0x8000
    special[5, :] = np.random.default_rng(9).integers(0, 0x80, 128)        # subnormals only
    special[6, 7] = 0x7F7F                                                  # largest finite
    special[7, :] = 0x3F80
    rows.append(special)
    X = np.concatenate(rows)
    T = X.shape[0] // 8 * 8
    X = X[:T].reshape(T // 8, 8 * 128)            # H = 1024
    x = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev)
    xq, xs = moe.quant_act(x)
    torch.cuda.synchronize()
    rq, rs = quant_act_ref(X)
    assert np.array_equal(xs.cpu().numpy(), rs)
    assert np.array_equal(xq.cpu().numpy(), rq)


# ----------------------------------------------------------------------------- planner

@pytest.mark.parametrize("T,K,E,seed", [(1, 1, 1, 0), (7, 8, 384, 1), (64, 2, 8, 2), (256, 8, 384, 3),
                                        (255, 3, 5, 4), (300, 8, 4096, 5), (4096, 8, 384, 6), (5000, 7, 64, 7),
                                        (50, 64, 100, 8), (3000, 16, 384, 9)])
def test_plan_random(dev, T, K, E, seed):
    ids = np.random.default_rng(seed).integers(0, E, (T, K)).astype(np.int32)
    p = moe.plan(torch.from_numpy(ids).to(dev), E, 256, 256)
    torch.cuda.synchronize()
    check_plan(p, ids, E)


@pytest.mark.parametrize("name", ["tiny", "decode7", "decode256", "prefill32k"])
def test_plan_workloads(dev, name):
    w = WORKLOADS[name]
    ids, _ = make_routing(w)
    p = moe.plan(torch.from_numpy(ids).to(dev), w.E, w.H, w.I)
    torch.cuda.synchronize()
    check_plan(p, ids, w.E)


@pytest.mark.parametrize("T", [100, 3000])
def test_plan_invalid_ids_dropped(dev, T):
    rng = np.random.default_rng(T)
    ids = rng.integers(0, 16, (T, 4)).astype(np.int32)
    bad = rng.random(ids.shape) < 0.1
    ids[bad] = rng.choice([-1, 16, 1 << 30, -(1 << 30)], bad.sum())
    p = moe.plan(torch.from_numpy(ids).to(dev), 16, 256, 256)
    torch.cuda.synchronize()
    check_plan(p, ids, 16)


def test_plan_empty(dev):
    p = moe.plan(torch.zeros((0, 8), dtype=torch.int32, device=dev), 32, 256, 256)
    torch.cuda.synchronize()
    assert not p.expert_offsets.cpu().numpy().any() and int(p.status.cpu()[0]) == 0


# ----------------------------------------------------------------------------- FFN, small shapes

@pytest.mark.parametrize("small_max", [0, 1, 10 ** 6])
def test_ffn_tiny(dev, small_max):
    """Tiny config (64 tokens, H 256, 8 experts, I 512, top-2) in full, with the
    default small/large split, everything on the large-M path, everything small."""
    inp = make_inputs("tiny").to(dev)
    p, (y, dbg) = run_path(inp, small_max=small_max)
    check_plan(p, inp.topk_ids.cpu().numpy(), inp.wl.E)
    check_ffn(inp, p, y, dbg, label=f"tiny small_max={small_max}")


@pytest.mark.parametrize("wl", [
    dict(base="tiny"),
    dict(base="tiny", T=700, H=1024, I=512, E=2, K=1, seed=56, weight_seed=56),    # 256-row items + remainders
    dict(base="tiny", T=400, H=256, I=384, E=1, K=1, seed=52, weight_seed=52),     # few-K W2
])
def test_tilings_agree_bit_for_bit(dev, wl):
    """The small-M tiles (weights on the MFMA's A side, 16 tokens per tile), the
    128-row and the 256 x 256 large-M tiles all sum each dot product over
    ascending 128-K steps with the same instruction, so y and the SwiGLU codes
    are identical bit for bit whichever tiling the split sends an expert to."""
    base = wl.pop("base")
    inp = make_inputs(scaled(base, name="tilings", **wl) if wl else base).to(dev)
    outs = []
    for small_max in (0, 1, 10 ** 6):
        p, (y, dbg) = run_path(inp, small_max=small_max)
        rows = p.pair_rows.cpu().numpy()
        order = rows[rows >= 0]
        outs.append((u16(y), dbg["h_q"].cpu().numpy()[order], dbg["h_s"].cpu().numpy()[order]))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("T,H,I,E,K,seed,small_max", [
    (1, 128, 128, 1, 1, 41, 0),        # degenerate: one token, one expert
    (33, 384, 384, 5, 3, 42, 0),       # ragged: odd T, H and I not multiples of 256
    (130, 640, 256, 3, 2, 43, 0),      # experts with > 128 rows (several large tiles + a tail)
    (17, 256, 1152, 40, 8, 44, 0),     # many experts, I = 9 * 128
    # small_max 1 sends experts with 2+ rows to the large-M path: odd K-step
    # counts (W2 K = 1152 and 384: 9 and 3 steps), a count that ends inside a
    # weight-scale chunk (W13 K = 1280: 10 steps), 17 steps
    (130, 256, 1152, 3, 2, 45, 1),
    (200, 1280, 384, 4, 2, 46, 1),
    (150, 256, 2176, 2, 1, 47, 1),
    # 256-row items (256 x 256 tiles need a K-step count divisible by 4; other counts
    # run those items as two 128-row halves): one full item + a 44-row remainder
    # item; two experts with full items and remainders (W13 on halves, W2 with 6
    # steps on halves); a second item with 144 of 256 rows (W2 on 256 x 256 tiles);
    # W2 with 3 K steps; 16 W13 K steps (the weight-scale chunk buffers rotate); 6
    # W13 K steps (activation scale rows not 4-byte aligned, a partial last scale
    # chunk); 144-row second items and remainders with both GEMMs on 256 x 256 tiles
    (300, 512, 512, 1, 1, 48, 0),
    (700, 256, 768, 2, 1, 49, 0),
    (400, 256, 512, 1, 1, 51, 0),
    (400, 256, 384, 1, 1, 52, 0),
    (300, 2048, 1024, 1, 1, 53, 0),
    (300, 768, 256, 1, 1, 54, 0),
    (400, 512, 512, 1, 1, 55, 0),
    (700, 1024, 512, 2, 1, 56, 0),
    # W2 with 1..3 K steps on the few-K kernel (routed rows kept in LDS, runs of
    # 256-column blocks; H 1280 = 5 blocks -> runs of 3 and 2): one expert with a
    # 256-row item and a remainder, several experts with 128-row items only
    (300, 512, 128, 1, 1, 57, 0),
    (400, 1280, 256, 3, 2, 58, 0),
    (600, 1280, 384, 2, 1, 59, 0),
    # top-k above 8: the combine adds picks in batches of 8 (K 16: two full
    # batches; K 64, the largest the library takes: eight), the planner ranks
    # 16 or 64 picks per token
    (40, 256, 256, 64, 16, 64, 0),
    (9, 256, 256, 80, 64, 65, 0),
    (70, 512, 384, 40, 12, 66, 0),
    # 4096 experts, the most the library takes (multi-block plan, expert ids past
    # 2^11 in every list and offset)
    (600, 128, 128, 4096, 4, 67, 0),
])
def test_ffn_shapes(dev, T, H, I, E, K, seed, small_max):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"s{seed}")
    inp = make_inputs(wl).to(dev)
    p, (y, dbg) = run_path(inp, small_max=small_max)
    check_ffn(inp, p, y, dbg, label=f"shape {T}x{H} I{I} E{E} K{K} small_max={small_max}")


@pytest.mark.parametrize("T,H,I,E,K,Is,seed,small_max", [
    (1, 128, 128, 1, 1, 128, 51, 0),      # degenerate: one token, one expert, one shared tile
    (33, 256, 256, 5, 3, 128, 52, 0),     # ragged token tile (33 of 128 rows)
    (130, 384, 128, 4, 2, 256, 53, 1),    # H = 3 * 128: the shared W2 tile's second half is masked
    (200, 1280, 384, 4, 2, 384, 54, 1),   # odd K-step count in the shared W2 (Is = 3 * 128)
    (130, 384, 128, 4, 2, 512, 55, 1),    # Is = 512: the generic shared W2 tiles, H/128 odd (masked half)
])
def test_ffn_shared_shapes(dev, T, H, I, E, K, Is, seed, small_max):
    """Routed experts plus the dense FP8 shared expert (128 x 128 block scales):
    y, the shared SwiGLU codes and scales against the oracle."""
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, Is=Is, seed=seed, weight_seed=seed, name=f"sh{seed}")
    inp = make_inputs(wl).to(dev)
    assert inp.shared is not None
    p, (y, dbg) = run_path(inp, small_max=small_max)
    check_ffn(inp, p, y, dbg, label=f"shared {T}x{H} I{I} Is{Is} E{E} K{K}")


@pytest.mark.parametrize("T,H,I,E,K,seed", [
    (3, 16384, 256, 4, 2, 60),     # H at the small-M limit (W13 scale runs of 8 KB per wave in LDS)
    (2, 256, 16384, 2, 1, 61),     # I at the small-M limit (W2 scale runs of 4*I bytes)
    (300, 8192, 256, 1, 1, 62),    # H/128 = 64 K steps, the most the large-M tiles keep scales for
    (300, 8320, 256, 1, 1, 63),    # 65 K steps: the large-M tiles do not apply, the small-M kernels walk the items
])
def test_ffn_size_limits(dev, T, H, I, E, K, seed):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"lim{seed}")
    inp = make_inputs(wl).to(dev)
    p, (y, dbg) = run_path(inp)
    check_ffn(inp, p, y, dbg, label=f"limit {T}x{H} I{I} E{E} K{K}")


def test_ffn_empty_batch(dev):
    """T = 0 is a valid no-op for both calls."""
    wl = scaled("tiny", T=1, name="empty")
    W = moe.pack_weights(make_inputs(wl).to(dev).weights)
    ids = torch.zeros((0, wl.K), dtype=torch.int32, device=dev)
    p = moe.plan(ids, wl.E, wl.H, wl.I)
    y = moe.ffn(torch.zeros((0, wl.H), dtype=torch.bfloat16, device=dev),
                torch.zeros((0, wl.K), dtype=torch.float32, device=dev), p, W)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, wl.H)


def test_ffn_invalid_ids(dev):
    inp = make_inputs("tiny").to(dev)
    ids = inp.topk_ids.clone()
    ids[::5, 1] = -3
    ids[3, 0] = 99
    inp.topk_ids = ids
    p, (y, dbg) = run_path(inp)
    assert int(p.status.cpu()[0]) == int((ids < 0).sum() + (ids >= inp.wl.E).sum())
    check_ffn(inp, p, y, dbg, label="tiny with dropped ids")


@pytest.mark.parametrize("name,shared,flags", [("decode256", False, 0), ("decode7", False, 0),
                                                ("decode7", False, moe.FLAG_DECODE_CHAIN),
                                                ("tp8small", True, moe.FLAG_DECODE_CHAIN)])
def test_ffn_bitwise_repeatable_whatever_the_workspace_holds(dev, full_weights, name, shared, flags):
    """Identical inputs give bitwise identical outputs, and nothing in the workspace
    needs initializing: the FFN runs four times with its workspace pre-filled with
    different byte patterns and y is compared bit for bit. decode256 and decode7 on
    the separate kernels, decode7 on the persistent chain, and the chain with the
    shared expert."""
    if shared:
        wl = scaled("tiny", T=40, H=1024, I=512, E=6, K=4, Is=256, seed=81, weight_seed=81, name="rep_shared")
        inp = make_inputs(wl).to(dev)
        W = moe.pack_weights(inp.weights)
    else:
        inp = _full_inputs(name, dev, full_weights)
        W = moe.pack_weights(full_weights)
    w = inp.wl
    p = moe.plan(inp.topk_ids, w.E, w.H, w.I, Is=w.Is if shared else 0, flags=flags)
    ws = torch.empty(moe.ffn_workspace_bytes(p.dims), dtype=torch.uint8, device=dev)
    ys = []
    for fill in (0x00, 0xFF, 0x55, 0x7B):
        ws.fill_(fill)
        ys.append(u16(moe.ffn(inp.x, inp.topk_weights, p, W, shared=inp.shared if shared else None, ws=ws)))
    for y in ys[1:]:
        assert np.array_equal(y, ys[0])
    del W


@pytest.mark.parametrize("wl", [
    dict(base="tiny"),
    dict(base="tiny", T=40, H=1024, I=512, E=6, K=4, Is=256, seed=82, weight_seed=82),   # + shared expert
    dict(base="tiny", T=300, H=512, I=512, E=1, K=1, seed=83, weight_seed=83),           # 256-row + 128-row items
    dict(base="tiny", T=130, H=384, I=1152, E=3, K=2, seed=84, weight_seed=84),          # H/256 odd, I 9 x 128
    dict(base="tiny", T=3, H=16384, I=256, E=4, K=2, seed=85, weight_seed=85),           # H at the small-M limit
    dict(base="tiny", T=24, H=512, I=256, E=48, K=16, seed=86, weight_seed=86),          # top-16, 384 pairs
])
def test_decode_chain_matches_separate_launches(dev, wl):
    """MOE_FLAG_DECODE_CHAIN (one persistent launch of W13, W2 and the combine,
    synchronized by per-expert and per-column-block counters) gives bitwise the
    separate launches' y and SwiGLU codes, also with dropped picks and with every
    pick dropped."""
    base = wl.pop("base")
    wl = scaled(base, name="chain", **wl) if wl else WORKLOADS[base]
    inp = make_inputs(wl).to(dev)
    for drop in (None, "some", "all"):
        if drop == "some":
            inp.topk_ids = inp.topk_ids.clone()
            inp.topk_ids[::3, 0] = -1
        elif drop == "all":
            inp.topk_ids = torch.full_like(inp.topk_ids, wl.E + 5)
        outs = []
        for flags in (0, moe.FLAG_DECODE_CHAIN):
            p, (y, dbg) = run_path(inp, flags=flags)
            rows = p.pair_rows.cpu().numpy()
            order = np.sort(rows[rows >= 0])
            keys = ("h_q", "h_s") + (("sh_q", "sh_s") if inp.shared is not None else ())
            outs.append([u16(y)] + [dbg[k].cpu().numpy()[order] if k[0] == "h" else dbg[k].cpu().numpy()
                                    for k in keys])
        for a, b in zip(*outs):
            assert np.array_equal(a, b), drop


def test_decode_chain_decode7_parity(dev, full_weights):
    """The 7-token verify through the persistent chain, every token against the oracle."""
    inp = _full_inputs("decode7", dev, full_weights)
    p, (y, dbg) = run_path(inp, flags=moe.FLAG_DECODE_CHAIN)
    check_ffn(inp, p, y, dbg, label="decode7 chain")


def test_ffn_deterministic_and_token_permutation(dev):
    inp = make_inputs(scaled("tiny", T=200, E=16, K=4, name="perm")).to(dev)
    _, (y1, _) = run_path(inp)
    _, (y2, _) = run_path(inp)
    assert torch.equal(y1, y2)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(200)).to(dev)
    inp.x, inp.topk_ids, inp.topk_weights = inp.x[perm].contiguous(), inp.topk_ids[perm].contiguous(), \
        inp.topk_weights[perm].contiguous()
    _, (y3, _) = run_path(inp)
    assert torch.equal(y3, y1[perm])


# ----------------------------------------------------------------------------- FFN, full sizes

@pytest.fixture(scope="module")
def full_weights(dev):
    """The 384-expert MXFP4 weight set of the H 7168 / I 3072 workloads (13.5 GB),
    generated on the GPU once for this module."""
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


def test_ffn_decode7_full(dev, full_weights):
    """7-token verify at full size, every token checked against the oracle."""
    inp = _full_inputs("decode7", dev, full_weights)
    p, (y, dbg) = run_path(inp)
    check_plan(p, inp.topk_ids.cpu().numpy(), inp.wl.E)
    check_ffn(inp, p, y, dbg, label="decode7 full")


@pytest.mark.timeout(600)
def test_ffn_decode256_full(dev, full_weights):
    """32 requests x 8 speculative positions at full size: every token and pair."""
    inp = _full_inputs("decode256", dev, full_weights)
    p, (y, dbg) = run_path(inp)
    check_plan(p, inp.topk_ids.cpu().numpy(), inp.wl.E)
    check_ffn(inp, p, y, dbg, label="decode256 full")


@pytest.mark.timeout(900)
def test_ffn_prefill32k_full(dev, full_weights):
    """The 32K prefill chunk at full size: all 32,768 tokens and 262,144 pairs
    (every 256-row and 128-row work item, every column block)."""
    inp = _full_inputs("prefill32k", dev, full_weights)
    p, (y, dbg) = run_path(inp)
    check_plan(p, inp.topk_ids.cpu().numpy(), inp.wl.E)
    say("[prefill32k full] GPU done, running the oracle on every token")
    check_ffn(inp, p, y, dbg, label="prefill32k full")


@pytest.mark.timeout(600)
def test_ffn_tp8rank32k_full(dev):
    """One TP8 rank of the 32K prefill (routed I 384 slice + the FP8 shared
    expert): all tokens and pairs."""
    import time
    t = time.time()
    inp = make_inputs("tp8rank32k", weights=False).to(dev)
    inp.weights = make_expert_weights(inp.wl, dev)
    inp.shared = make_shared_weights(inp.wl, dev)
    torch.cuda.synchronize()
    say(f"[tp8rank32k weights] generated in {time.time() - t:.1f}s")
    p, (y, dbg) = run_path(inp)
    check_plan(p, inp.topk_ids.cpu().numpy(), inp.wl.E)
    check_ffn(inp, p, y, dbg, label="tp8rank32k full")


# ----------------------------------------------------------------------------- exact-shape tiling per GEMM

def _sized_routing(sizes, K, seed):
    """topk_ids [T, K] with exactly sizes[e] pairs routed to expert e (distinct
    experts per token are not required: duplicates are independent pairs)."""
    rng = np.random.default_rng(seed)
    ids = np.concatenate([np.full(m, e, dtype=np.int32) for e, m in enumerate(sizes)])
    rng.shuffle(ids)
    return torch.from_numpy(ids.reshape(-1, K).copy())


def _work_lists_ref(ids, E, small_max, t13, t2):
    """The planner's tile work lists written out from their definition, from the
    per-expert pair counts m: 16-row tiles (expert, 16 i) of the experts with
    1..small_max pairs, in expert order; for the larger experts, heaviest first (ties:
    lower id), 256-row items (expert, 256 i) for i < (m + 127) // 256, and one
    128-row item (expert, m - r) when the remainder r = m % 256 is 1..128, these
    ordered by r (ties: heavier, then lower id); the header: the three list lengths
    and how many 128-row items have at most t13 / t2 rows."""
    v = ids[(ids >= 0) & (ids < E)]
    cnt = np.bincount(v, minlength=E)
    small = [(e, 16 * i) for e in range(E) if 1 <= cnt[e] <= small_max for i in range(-(-cnt[e] // 16))]
    big = sorted((e for e in range(E) if cnt[e] > small_max), key=lambda e: (-cnt[e], e))
    xl = [(e, 256 * i) for e in big for i in range((cnt[e] + 127) // 256)]
    rem = {e: cnt[e] % 256 for e in big}
    with_rem = sorted((e for e in big if 1 <= rem[e] <= 128), key=lambda e: (rem[e], -cnt[e], e))
    large = [(e, cnt[e] - rem[e]) for e in with_rem]
    if not big:
        hdr = [len(small), 0, 0, 0, 0]
    else:
        hdr = [len(small), len(large), len(xl), sum(rem[e] <= t13 for e in with_rem),
               sum(rem[e] <= t2 for e in with_rem)]
    return small, large, xl, hdr


def _work_lists(p, T, K, E, small_max):
    """The lists as the plan workspace holds them: a 64-byte int32 header, then the
    small, 128-row and 256-row lists of {expert, first row} pairs, each region rounded
    up to 256 bytes and sized by the library's host-side bounds (written out here:
    min(P, E) small tiles, plus P / 16 when small_max > 16; min(P / (small_max + 1), E)
    large experts; min(P / 129, P / 256 + that) 256-row items)."""
    P = T * K
    sc = min(P, E) + (P // 16 if small_max > 16 else 0)
    big = min(P // (small_max + 1), E)
    lc = big
    al = lambda n: (n + 255) // 256 * 256
    o_small = 256
    o_large = o_small + al(8 * max(sc, 1))
    o_xl = o_large + al(8 * max(lc, 1))
    ws = p.ws.cpu().numpy()
    hdr = ws[:20].view(np.int32).tolist()
    lst = lambda o, n: [tuple(r) for r in ws[o:o + 8 * n].view(np.int32).reshape(-1, 2).tolist()]
    return lst(o_small, hdr[0]), lst(o_large, hdr[1]), lst(o_xl, hdr[2]), hdr


@pytest.mark.parametrize("case", ["ties", "prefill32k", "small_max1", "decode7", "e4096"])
def test_plan_work_lists_match_definition(dev, case):
    """Every tile work list and header count of the plan equals the definition above,
    exactly: expert sizes with ties in pair count and in remainder, a 32K-token routing
    (384 experts, every one above small_max), many large experts at small_max 1, a
    decode step (no large expert: empty large-M lists), and 4096 experts of about 20
    pairs each (thousands of ties on both sides of small_max)."""
    t13, t2 = 48, -1
    if case == "ties":
        sizes = [300, 300, 17, 17, 0, 600, 129, 256, 40, 40, 513, 5, 16, 3, 812, 44, 300]
        ids = _sized_routing(sizes, 1, 131).numpy()
        E, K, sm = len(sizes), 1, 16
    elif case == "prefill32k":
        ids = make_inputs("prefill32k", weights=False).topk_ids.numpy()
        E, K, sm = 384, 8, 16
        t13, t2 = 16, -1
    elif case == "small_max1":
        rng = np.random.default_rng(132)
        E, K, sm = 64, 4, 1
        ids = rng.integers(-2, E + 2, (700, K)).astype(np.int32)
    elif case == "decode7":
        ids = make_inputs("decode7", weights=False).topk_ids.numpy()
        E, K, sm = 384, 8, 16
    else:
        rng = np.random.default_rng(133)
        E, K, sm = 4096, 4, 16
        ids = rng.integers(0, E, (20000, K)).astype(np.int32)
    T = ids.shape[0]
    P = T * K
    p = moe.plan(torch.from_numpy(ids).to(dev), E, 1024, 512, small_max=sm, tile_w13=t13, tile_w2=t2)
    torch.cuda.synchronize()
    eff = (128, 128) if P <= 512 else (t13 if t13 > 0 else 0, t2 if t2 > 0 else 0)
    ref = _work_lists_ref(ids, E, sm, *eff)
    got = _work_lists(p, T, K, E, sm)
    for name, a, b in zip(("small", "large", "xl"), got[:3], ref[:3]):
        assert a == b, (case, name, len(a), len(b), [i for i in range(min(len(a), len(b))) if a[i] != b[i]][:5])
    assert got[3][:5] == ref[3], (case, got[3][:5], ref[3])
    check_plan(p, ids, E)


def test_tile_choice_per_gemm_is_bitwise_neutral(dev):
    """Expert sizes covering every item kind above the decode fold (P > 512): a
    remainder of 44 and 88 rows after 256-row items, whole experts of 17, 20 and 100
    rows (one 128-row item each), a 129-row expert and a 256 + 144-row one (partial
    256-row items), and a 256-row expert with no remainder. Whatever prefix of the
    128-row items (sorted by rows) each GEMM walks as 16-row tiles, y is identical
    bit for bit, also with the workspace (which then holds the SwiGLU rows and the
    per-pair rows) and y filled with other bytes beforehand (0xFF is NaN as fp16: a
    row that no kernel wrote would show), and so are the SwiGLU codes; the planner's
    per-GEMM counts follow the thresholds; the result matches the oracle."""
    sizes = [300, 400, 20, 100, 129, 256, 17, 600]
    K = 2
    T = sum(sizes) // K
    P = T * K
    wl = scaled("tiny", T=T, H=1024, I=512, E=len(sizes), K=K, seed=121, weight_seed=121, name="tiles")
    inp = make_inputs(wl).to(dev)
    inp.topk_ids = _sized_routing(sizes, K, 121).to(dev)
    packed = moe.pack_weights(inp.weights)
    rems = sorted(m % 256 for m in sizes if m > 16 and 1 <= m % 256 <= 128)
    assert rems == [17, 20, 44, 88, 100]
    ids = inp.topk_ids.cpu().numpy()
    configs = ((-1, -1), (128, 128), (44, 20), (20, 100), (1, 99))
    cnt = lambda t: sum(r <= t for r in rems) if t > 0 else 0
    ref_plan = plan_ref(ids, wl.E)
    ys, codes, labels, plan_ok = [], [], [], []
    for fill in (0xFF, 0x00, 0x5A):
        for t13, t2 in configs:
            p = moe.plan(inp.topk_ids, wl.E, wl.H, wl.I, tile_w13=t13, tile_w2=t2)
            ws = torch.full((moe.ffn_workspace_bytes(p.dims),), fill, dtype=torch.uint8, device=dev)
            y = torch.full((T, wl.H), fill * 0x101 - (0x10000 if fill >= 0x80 else 0), dtype=torch.int16,
                           device=dev).view(torch.bfloat16)
            moe.ffn(inp.x, inp.topk_weights, p, packed, ws=ws, y=y)
            torch.cuda.synchronize()
            hdr = p.ws[:20].view(torch.int32).cpu().numpy()
            assert hdr[1] == len(rems) and hdr[3] == cnt(t13) and hdr[4] == cnt(t2), (t13, t2, hdr)
            plan_ok.append(np.array_equal(p.sorted_pairs.cpu().numpy()[:P], ref_plan["sorted_pairs"]) and
                           np.array_equal(p.pair_rows.cpu().numpy()[:P], ref_plan["pair_rows"]) and
                           np.array_equal(p.expert_offsets.cpu().numpy(), ref_plan["expert_offsets"]))
            ys.append(u16(y))
            labels.append(f"fill {fill:#x} tiles w13<={t13} w2<={t2}")
            if fill == 0x00:
                y2, dbg = moe.ffn(inp.x, inp.topk_weights, p, packed, debug=True)
                torch.cuda.synchronize()
                rows = p.pair_rows.cpu().numpy()
                order = rows[rows >= 0]
                codes.append((dbg["h_q"].cpu().numpy()[order], dbg["h_s"].cpu().numpy()[order]))
                if t13 == 44:
                    check_ffn(inp, p, y2, dbg, label=labels[-1])
    mismatch = [i for i in range(1, len(ys)) if not np.array_equal(ys[0], ys[i])]
    if mismatch:
        ref = ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **inp.weights)["y"]
        sc = np.abs(ref).max()
        for i, (lab, a) in enumerate(zip(labels, ys)):
            err = np.abs(bf16_to_f64(a) - ref) / sc
            bad = np.nonzero(~(err.max(axis=1) <= MAX_REL))[0]
            cols = np.nonzero(~(err[bad] <= MAX_REL).all(axis=0))[0] if bad.size else np.zeros(0, int)
            say(f"[tiles] '{lab}': plan arrays {'ok' if plan_ok[i] else 'DIFFER from plan_ref'}; tokens off the "
                f"oracle {bad.size} {bad[:8].tolist()} (experts {ids[bad[:8]].tolist()}), columns {cols.size} "
                f"[{cols.min() if cols.size else '-'}..{cols.max() if cols.size else '-'}]")
    assert not mismatch, [labels[i] for i in mismatch]
    for c in codes[1:]:
        assert np.array_equal(codes[0][0], c[0]) and np.array_equal(codes[0][1], c[1])
