"""Pins for the oracle's NVFP4 statement (oracle.moe.ffn_ref_nvfp4, dequant_nvfp4,
oracle.envelope.routed_swiglu_envelope_nvfp4).

* brute force: oracle/brute.py's NVFP4 mode (weights as exact fractions E2M1 x
  E4M3 x tensor scale, fsum dots, bisection bf16 rounding) agrees on every bf16
  SwiGLU output and on y to float64 rounding;
* dequantization: against the fraction decode on random codes and scales, and the
  special case of unit block scales, where NVFP4 reduces to the plain E2M1 grid;
* exactness of the float64 GEMMs at H = 7168 with bf16 activations;
* invariants: a power-of-two W2 tensor scale scales y exactly; a power-of-two
  block-scale change with the opposite tensor-scale change leaves y unchanged;
* the generator's weights decode to within half an E2M1 step of the float weights;
* the envelope's exact values are those of fsum dots, and it covers emulated
  hardware dot products.
"""

import math

import numpy as np
import pytest
import torch

from oracle import envelope as env
from oracle.brute import brute_ref_nvfp4, e2m1, e4m3, nvfp4_row
from oracle.formats import E2M1_VALUES, E4M3_VALUES, bf16_to_f64
from oracle.moe import dequant_mxfp4, dequant_nvfp4, ffn_ref_nvfp4
from synth import make_expert_weights, make_inputs, scaled
from synth.workloads import _pack_nvfp4


def _bits(x):
    return x.view(torch.int16).numpy().view(np.uint16)


def _nv_inputs(T, H, I, E, K, seed):
    wl = scaled("tiny", T=T, H=H, I=I, E=E, K=K, seed=seed, weight_seed=seed, name=f"nv{seed}")
    inp = make_inputs(wl, weights=False)
    return inp, make_expert_weights(wl, fmt="nvfp4")


@pytest.mark.parametrize("T,H,I,E,K,seed", [(3, 256, 256, 3, 2, 91), (2, 128, 128, 1, 1, 92)])
def test_nvfp4_ref_equals_bruteforce(T, H, I, E, K, seed):
    inp, W = _nv_inputs(T, H, I, E, K, seed)
    ids = inp.topk_ids.numpy().copy()
    if E > 1:
        ids[0, 1] = -1
    r = ffn_ref_nvfp4(inp.x, ids, inp.topk_weights, **W)
    b = brute_ref_nvfp4(_bits(inp.x), ids, inp.topk_weights.numpy(), **{k: v.numpy() for k, v in W.items()})
    assert np.array_equal(r["h_q"][r["valid"]], b["h_q"][r["valid"]])
    np.testing.assert_allclose(r["y"], b["y"], rtol=1e-13, atol=1e-15 * np.abs(b["y"]).max())


def test_dequant_nvfp4_against_fractions_and_unit_scales():
    rng = np.random.default_rng(93)
    codes = rng.integers(0, 256, (6, 32), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (6, 4), dtype=np.uint8)          # every non-negative finite E4M3
    scales[0, 0] = 0                                                 # zero block
    scales[1, 1] = 0x01                                              # smallest subnormal
    d = dequant_nvfp4(codes, scales).numpy()
    for n in range(6):
        assert [float(v) for v in nvfp4_row(codes[n], scales[n], 1.0)] == d[n].tolist()
    one = np.full((6, 4), 0x38, dtype=np.uint8)                      # E4M3 1.0
    assert E4M3_VALUES[0x38] == 1.0
    plain = dequant_mxfp4(codes, np.full((6, 2), 127, dtype=np.uint8)).numpy()
    assert np.array_equal(dequant_nvfp4(codes, one).numpy(), plain)
    assert e2m1(0xF) == -6 and e4m3(0x7E) == 448


def test_nvfp4_float64_gemm_is_exact_at_full_hidden_size():
    wl = scaled("decode7", E=1, T=8, I=128, full_I=0, weight_seed=94, seed=94, name="nvex")
    W = make_expert_weights(wl, fmt="nvfp4")
    xh = bf16_to_f64(_bits(make_inputs(wl, weights=False).x))
    Wd = dequant_nvfp4(W["w13"][0], W["w13_s"][0]).numpy()
    blas = xh @ Wd.T
    for t in range(xh.shape[0]):
        for n in range(0, Wd.shape[0], 37):
            assert blas[t, n] == math.fsum(xh[t] * Wd[n])


def test_nvfp4_tensor_scale_invariants():
    inp, W = _nv_inputs(16, 256, 256, 4, 2, 95)
    base = ffn_ref_nvfp4(inp.x, inp.topk_ids, inp.topk_weights, **W)
    W2 = dict(W, w2_gs=W["w2_gs"] * 4)
    assert np.array_equal(ffn_ref_nvfp4(inp.x, inp.topk_ids, inp.topk_weights, **W2)["y"], 4 * base["y"])
    # block scales one binade down (E4M3 exponent field - 1, which keeps them
    # normal) and the tensor scale doubled: the same weights, the same result
    s = W["w13_s"].clone()
    field = (s >> 3) & 0xF
    assert bool((field >= 2).all())
    W3 = dict(W, w13_s=s - 8, w13_gs=W["w13_gs"] * 2)
    r3 = ffn_ref_nvfp4(inp.x, inp.topk_ids, inp.topk_weights, **W3)
    assert np.array_equal(r3["h_q"], base["h_q"]) and np.array_equal(r3["y"], base["y"])


def test_nvfp4_generator_rounds_to_the_grid():
    """_pack_nvfp4 (input generation) decodes, with its tensor scale, to within
    half an E2M1 step of the float weights (step at most 2 x block scale), and its
    largest block scale sits at the top of the E4M3 range."""
    g = torch.Generator().manual_seed(96)
    wf = torch.randn((64, 256), generator=g) * 0.02
    codes, scales, gs = _pack_nvfp4(wf)
    deq = dequant_nvfp4(codes, scales).numpy() * gs
    step = np.repeat(E4M3_VALUES[scales.numpy().astype(np.int64)] * gs, 16, axis=-1) * 2.0
    assert (np.abs(deq - wf.double().numpy()) <= step / 2 + 1e-12).all()
    assert E4M3_VALUES[int(scales.max())] >= 400


def test_nvfp4_envelope_values_and_bound():
    rng = np.random.default_rng(97)
    T, H, I = 3, 256, 128
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xv = bf16_to_f64(x)
    codes, scales, gs = _pack_nvfp4(torch.randn((2 * I, H), generator=torch.Generator().manual_seed(11)) * 0.02)
    tok = np.array([0, 2, 1, 2, 0])
    col = np.array([3, 127, 0, 90, 64])
    h, err = env.routed_swiglu_envelope_nvfp4(x, codes.numpy(), scales.numpy(), gs, I, tok, col)
    Wd = dequant_nvfp4(codes, scales).numpy()
    for i in range(tok.size):
        g = gs * math.fsum(xv[tok[i]] * Wd[col[i]])
        u = gs * math.fsum(xv[tok[i]] * Wd[I + col[i]])
        assert h[i] == g / (1 + math.exp(-g)) * u
        emu = [float(np.float32(gs) * np.float32(env.emulate_bf16_dot(xv[tok[i]][None], Wd[c][None])[0]))
               for c in (col[i], I + col[i])]
        g32, u32 = emu
        e = np.float32(np.exp2(np.float32(np.float32(g32) * np.float32(-1.4426950408889634))))
        h32 = float(np.float32(np.float32(np.float32(g32) * (np.float32(1) / (np.float32(1) + e))) * np.float32(u32)))
        assert abs(h32 - h[i]) <= err[i]
        assert err[i] < abs(h[i]) * 2.0 ** -6 + 1e-9
