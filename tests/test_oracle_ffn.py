"""Pins for oracle.ffn_ref (the whole FFN in float64).

* brute force: oracle/brute.py (own codecs, per-token / per-pick loops, fsum)
  must agree on every SwiGLU code and on y to float64 rounding of the final sum;
* exactness of the float64 GEMMs: BLAS dot products equal math.fsum of the
  exact products at the real hidden size (7168) and weight statistics;
* invariants: uniform gating gives the mean of the single-expert outputs, a
  token permutation permutes y, relabelling experts changes nothing, K = 1
  reduces to one dense quantized SwiGLU FFN, the MoE-TP slices of the
  intermediate dimension add up to the unsliced result ("Pushing the Limits of
  Serving DeepSeek-V4-Pro", §3.1), zero input gives zero output, y is linear in
  the routing weights, dropped (out-of-range) picks contribute nothing.
"""

import math

import numpy as np
import pytest
import torch

from oracle.brute import brute_ref
from oracle.formats import dequantize_blocks
from oracle.moe import dequant_mxfp4, ffn_ref, ffn_ref_dense_single, quant_act_ref
from synth import make_expert_weights, make_inputs, scaled


def _np(d):
    return {k: v.numpy() for k, v in d.items()}


def _bits(x):
    return x.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,H,I,E,K,Is,seed", [
    (3, 256, 256, 3, 2, 0, 11),
    (2, 128, 128, 4, 3, 128, 12),
    (4, 128, 256, 1, 1, 0, 13),
])
def test_ffn_ref_equals_bruteforce(T, H, I, E, K, Is, seed):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, Is=Is, seed=seed, weight_seed=seed, name="b")
    inp = make_inputs(wl)
    ids = inp.topk_ids.numpy().copy()
    if E > 1:
        ids[0, 0] = E + 3          # an out-of-range id: dropped by both
    r = ffn_ref(inp.x, ids, inp.topk_weights, **inp.weights, shared=inp.shared)
    b = brute_ref(_bits(inp.x), ids, inp.topk_weights.numpy(), **_np(inp.weights),
                  shared=_np(inp.shared) if inp.shared else None)
    assert np.array_equal(r["h_q"][r["valid"]], b["h_q"][r["valid"]])
    assert np.array_equal(r["h_s"][r["valid"]], b["h_s"][r["valid"]])
    np.testing.assert_allclose(r["y"], b["y"], rtol=1e-13, atol=1e-15 * np.abs(b["y"]).max())


def test_w13_float64_gemm_is_exact_at_full_hidden_size():
    """The exactness the oracle relies on: BLAS float64 = math.fsum of exact
    products, at H = 7168 with N(0,1) activations and N(0, 0.02) MXFP4 weights."""
    wl = scaled("decode7", E=1, T=8, I=128, full_I=0, weight_seed=77, seed=77, name="ex")
    W = make_expert_weights(wl, "cpu")
    inp_x = make_inputs(wl, weights=False).x
    xq, xs = quant_act_ref(inp_x)
    xh = dequantize_blocks(xq, xs)
    Wd = dequant_mxfp4(W["w13"][0], W["w13_s"][0]).numpy()
    blas = xh @ Wd.T
    for t in range(xh.shape[0]):
        for n in range(0, Wd.shape[0], 37):
            assert blas[t, n] == math.fsum(xh[t] * Wd[n])


@pytest.fixture(scope="module")
def small():
    wl = scaled("tiny", T=32, H=256, I=512, E=6, K=2, seed=21, weight_seed=21, name="s")
    return make_inputs(wl)


def test_uniform_gating_is_mean_of_experts(small):
    ids = small.topk_ids.numpy()
    w = np.full(ids.shape, 0.5, dtype=np.float32)
    y = ffn_ref(small.x, ids, w, **small.weights)["y"]
    one = np.ones((ids.shape[0], 1), dtype=np.float32)
    y0 = ffn_ref(small.x, ids[:, :1], one, **small.weights)["y"]
    y1 = ffn_ref(small.x, ids[:, 1:], one, **small.weights)["y"]
    assert np.array_equal(y, 0.5 * y0 + 0.5 * y1)


def test_token_permutation(small):
    perm = np.random.default_rng(5).permutation(small.wl.T)
    r = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights)["y"]
    p = ffn_ref(small.x[perm], small.topk_ids[perm], small.topk_weights[perm], **small.weights)["y"]
    assert np.array_equal(p, r[perm])


def test_expert_relabel(small):
    E = small.wl.E
    relabel = np.random.default_rng(6).permutation(E)        # old id -> new id
    inv = np.argsort(relabel)
    W = {k: v[torch.from_numpy(inv)] for k, v in small.weights.items()}
    ids = relabel[small.topk_ids.numpy()]
    r = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights)["y"]
    p = ffn_ref(small.x, ids, small.topk_weights, **W)["y"]
    assert np.array_equal(p, r)


def test_k1_is_dense_single_expert(small):
    T = small.wl.T
    ids = np.full((T, 1), 3)
    y = ffn_ref(small.x, ids, np.ones((T, 1), np.float32), **small.weights)["y"]
    d = ffn_ref_dense_single(small.x, small.weights["w13"][3], small.weights["w13_s"][3],
                             small.weights["w2"][3], small.weights["w2_s"][3])
    assert np.array_equal(y, d)


def test_tp_slices_sum_to_full():
    """Split I = 1024 into 8 MoE-TP slices of 128: every quantization block of
    the SwiGLU output stays inside one slice, so the routed outputs add up."""
    wl = scaled("tiny", T=16, H=256, I=1024, E=4, K=2, seed=31, weight_seed=31, name="tp")
    inp = make_inputs(wl)
    W = inp.weights
    full = ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **W)["y"]
    I, R = 1024, 8
    s = I // R
    acc = np.zeros_like(full)
    for r in range(R):
        rows = torch.cat([torch.arange(r * s, (r + 1) * s), torch.arange(I + r * s, I + (r + 1) * s)])
        Wr = {"w13": W["w13"][:, rows], "w13_s": W["w13_s"][:, rows],
              "w2": W["w2"][:, :, r * s // 2:(r + 1) * s // 2].contiguous(),
              "w2_s": W["w2_s"][:, :, r * s // 32:(r + 1) * s // 32].contiguous()}
        acc += ffn_ref(inp.x, inp.topk_ids, inp.topk_weights, **Wr)["y"]
    np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-14 * np.abs(full).max())


def test_zero_input_and_linearity(small):
    z = torch.zeros_like(small.x)
    assert not ffn_ref(z, small.topk_ids, small.topk_weights, **small.weights)["y"].any()
    w1 = small.topk_weights.numpy()
    w2 = np.random.default_rng(8).random(w1.shape).astype(np.float32)
    a = ffn_ref(small.x, small.topk_ids, w1, **small.weights)["y"]
    b = ffn_ref(small.x, small.topk_ids, w2, **small.weights)["y"]
    c = ffn_ref(small.x, small.topk_ids, (w1.astype(np.float64) + w2).astype(np.float32), **small.weights)["y"]
    # w1 + w2 rounded to float32 differs from the exact sum by < 2^-24 relative
    np.testing.assert_allclose(c, a + b, rtol=1e-6, atol=1e-6 * np.abs(c).max())


def test_dropped_picks_contribute_nothing(small):
    ids = small.topk_ids.numpy().copy()
    ids[:, 1] = -1
    one = small.topk_weights.numpy().copy()
    r = ffn_ref(small.x, ids, one, **small.weights)
    r0 = ffn_ref(small.x, ids[:, :1], one[:, :1], **small.weights)
    assert np.array_equal(r["y"], r0["y"]) and not r["valid"][:, 1].any()


def test_token_subset_matches_full(small):
    full = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights)
    sub = [5, 0, 17]
    part = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights, tokens=sub)
    assert np.array_equal(part["y"], full["y"][sub])
    assert np.array_equal(part["h_q"], full["h_q"][sub])


# ----------------------------------------------------------------------------- bf16 activations (MXFP4A16)


@pytest.mark.parametrize("T,H,I,E,K,seed", [
    (3, 256, 256, 3, 2, 41),
    (4, 128, 128, 1, 1, 42),
])
def test_a16_ffn_ref_equals_bruteforce(T, H, I, E, K, seed):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name="b16")
    inp = make_inputs(wl)
    ids = inp.topk_ids.numpy().copy()
    if E > 1:
        ids[1, 0] = -1
    r = ffn_ref(inp.x, ids, inp.topk_weights, **inp.weights, act="bf16")
    b = brute_ref(_bits(inp.x), ids, inp.topk_weights.numpy(), **_np(inp.weights), act="bf16")
    assert r["h_q"].dtype == np.uint16 and r["x_q"] is None
    assert np.array_equal(r["h_q"][r["valid"]], b["h_q"][r["valid"]])
    np.testing.assert_allclose(r["y"], b["y"], rtol=1e-13, atol=1e-15 * np.abs(b["y"]).max())


def test_a16_bf16_nearest_matches_brute_on_edges():
    """Brute bf16 rounding (bisection over patterns, exact comparisons) against
    values placed on and around rounding boundaries, including ties both ways."""
    from oracle.brute import bf16_nearest
    from oracle.formats import f64_to_bf16_rne
    one = 1.0
    vals = [0.0, -0.0, one, one + 2 ** -8, one + 3 * 2 ** -8, one + 2 ** -8 + 2 ** -30, -(one + 2 ** -8),
            2 ** -126, 2 ** -133, 1.5 * 2 ** -133, 2.5 * 2 ** -133, 3.0e38, 1234.5678, -1e-20]
    assert [bf16_nearest(v) for v in vals] == [int(b) for b in f64_to_bf16_rne(np.array(vals))]
    assert bf16_nearest(one + 2 ** -8) == 0x3F80          # tie to even (down)
    assert bf16_nearest(one + 3 * 2 ** -8) == 0x3F82      # tie to even (up)
    assert bf16_nearest(-0.0) == 0x8000


def test_a16_float64_gemm_is_exact_at_full_hidden_size():
    """bf16 activations (8 significant bits) times MXFP4 values: the float64
    BLAS dots still equal math.fsum of the exact products at H = 7168."""
    from oracle.formats import bf16_to_f64
    wl = scaled("decode7", E=1, T=8, I=128, full_I=0, weight_seed=78, seed=78, name="ex16")
    W = make_expert_weights(wl, "cpu")
    xh = bf16_to_f64(_bits(make_inputs(wl, weights=False).x))
    Wd = dequant_mxfp4(W["w13"][0], W["w13_s"][0]).numpy()
    blas = xh @ Wd.T
    for t in range(xh.shape[0]):
        for n in range(0, Wd.shape[0], 37):
            assert blas[t, n] == math.fsum(xh[t] * Wd[n])


def test_a16_invariants(small):
    """K = 1 with weight 1 is the dense bf16 SwiGLU expert; uniform gating is the
    mean; dropped picks add nothing."""
    from oracle.formats import bf16_to_f64, f64_to_bf16_rne
    T, I = small.wl.T, small.wl.I
    W = small.weights
    y = ffn_ref(small.x, np.full((T, 1), 2), np.ones((T, 1), np.float32), **W, act="bf16")
    xh = bf16_to_f64(_bits(small.x))
    acc = xh @ dequant_mxfp4(W["w13"][2], W["w13_s"][2]).numpy().T
    g, u = acc[:, :I], acc[:, I:]
    h = bf16_to_f64(f64_to_bf16_rne(g / (1 + np.exp(-g)) * u))
    dense = h @ dequant_mxfp4(W["w2"][2], W["w2_s"][2]).numpy().T
    np.testing.assert_allclose(y["y"], dense, rtol=1e-13, atol=1e-15 * np.abs(dense).max())
    ids = small.topk_ids.numpy()
    half = np.full(ids.shape, 0.5, dtype=np.float32)
    one = np.ones((T, 1), dtype=np.float32)
    y2 = ffn_ref(small.x, ids, half, **W, act="bf16")["y"]
    y0 = ffn_ref(small.x, ids[:, :1], one, **W, act="bf16")["y"]
    y1 = ffn_ref(small.x, ids[:, 1:], one, **W, act="bf16")["y"]
    assert np.array_equal(y2, 0.5 * y0 + 0.5 * y1)
    d = ids.copy()
    d[:, 1] = E_OUT = small.wl.E + 5
    assert E_OUT > small.wl.E
    yd = ffn_ref(small.x, d, small.topk_weights, **W, act="bf16")
    y0w = ffn_ref(small.x, ids[:, :1], small.topk_weights.numpy()[:, :1], **W, act="bf16")
    assert np.array_equal(yd["y"], y0w["y"]) and not yd["valid"][:, 1].any()


def test_a16_differs_from_fp8_path(small):
    """The two activation modes are different computations: quantizing x to FP8
    moves y by far more than float64 rounding."""
    a = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights)["y"]
    b = ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights, act="bf16")["y"]
    rel = np.abs(a - b).max() / np.abs(b).max()
    assert 1e-4 < rel < 0.2


def test_a16_refuses_shared_and_unknown_modes(small):
    with pytest.raises(ValueError):
        ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights, act="fp16")
    sh = make_inputs(scaled("tiny", T=4, H=256, I=256, E=2, K=1, Is=128, seed=3, weight_seed=3, name="s16")).shared
    with pytest.raises(ValueError):
        ffn_ref(small.x, small.topk_ids, small.topk_weights, **small.weights, shared=sh, act="bf16")
