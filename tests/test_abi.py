"""The C-ABI library loads and exports every entry point the header declares, and
its host-side argument checks behave as documented. Nothing here launches GPU work."""

import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_weights_fp8_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mxfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(moe._SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for c in (0, -1, -2, -3, -4):
        assert moe.status_string(c).startswith("MOE_")
    assert "unknown" in moe.status_string(7)


@pytest.mark.parametrize("dims,code", [
    ((64, 256, 512, 8, 2), moe.MOE_OK),
    ((0, 7168, 3072, 384, 8), moe.MOE_OK),
    ((-1, 256, 512, 8, 2), moe.MOE_EINVAL),
    ((4, 256, 512, 0, 2), moe.MOE_EINVAL),
    ((4, 256, 512, 8, 0), moe.MOE_EINVAL),
    ((4, 256, 512, 4097, 2), moe.MOE_EINVAL),
    ((4, 200, 512, 8, 2), moe.MOE_EUNSUPPORTED),
    ((4, 256, 500, 8, 2), moe.MOE_EUNSUPPORTED),
    ((4, 16384, 16384, 8, 2), moe.MOE_OK),
    ((4, 16512, 512, 8, 2), moe.MOE_EUNSUPPORTED),   # H above the small-M kernels' LDS scale staging
    ((4, 256, 16512, 8, 2), moe.MOE_EUNSUPPORTED),
])
def test_validate(dims, code):
    assert moe.validate(moe.make_dims(*dims)) == code


def test_validate_flags():
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_DECODE_CHAIN)) == moe.MOE_OK
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_A16)) == moe.MOE_OK
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_A16 | moe.FLAG_DECODE_CHAIN)) == moe.MOE_OK
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_NVFP4)) == moe.MOE_OK
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=8)) == moe.MOE_EINVAL
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, flags=-1)) == moe.MOE_EINVAL


def test_validate_tile_fields():
    for v in (-1, 0, 1, 64, 128):
        assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, tile_w13=v, tile_w2=v)) == moe.MOE_OK
    for v in (-2, 129):
        assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, tile_w13=v)) == moe.MOE_EINVAL
        assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, tile_w2=v)) == moe.MOE_EINVAL


def test_validate_a16_limits():
    # no shared expert with bf16 activations
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, Is=128, flags=moe.FLAG_A16)) == moe.MOE_EUNSUPPORTED
    # bf16 rows addressed with 32-bit byte offsets: T*H and T*K*I below 2^30
    assert moe.validate(moe.make_dims(131072, 8192, 512, 8, 2, flags=moe.FLAG_A16)) == moe.MOE_EUNSUPPORTED
    assert moe.validate(moe.make_dims(131072, 8192, 512, 8, 2)) == moe.MOE_OK
    assert moe.validate(moe.make_dims(65536, 256, 2048, 8, 8, flags=moe.FLAG_A16)) == moe.MOE_EUNSUPPORTED
    assert moe.validate(moe.make_dims(65536, 256, 2048, 8, 4, flags=moe.FLAG_A16)) == moe.MOE_OK


def test_nvfp4_limits_follow_the_bf16_activation_path():
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, Is=128, flags=moe.FLAG_NVFP4)) == moe.MOE_EUNSUPPORTED
    assert moe.validate(moe.make_dims(65536, 256, 2048, 8, 8, flags=moe.FLAG_NVFP4)) == moe.MOE_EUNSUPPORTED
    d16 = moe.make_dims(4096, 1024, 512, 64, 8, flags=moe.FLAG_A16)
    dnv = moe.make_dims(4096, 1024, 512, 64, 8, flags=moe.FLAG_NVFP4)
    assert moe.ffn_workspace_bytes(dnv) == moe.ffn_workspace_bytes(d16)


def test_a16_workspace_holds_bf16_rows():
    d8 = moe.make_dims(4096, 1024, 512, 64, 8)
    d16 = moe.make_dims(4096, 1024, 512, 64, 8, flags=moe.FLAG_A16)
    assert moe.ffn_workspace_bytes(d16) - moe.ffn_workspace_bytes(d8) >= 4096 * 8 * 512


def test_validate_null_and_shared():
    assert moe.lib().moe_validate(None) == moe.MOE_EINVAL
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, Is=100)) == moe.MOE_EUNSUPPORTED
    assert moe.validate(moe.make_dims(4, 256, 512, 8, 2, Is=128)) == moe.MOE_OK


def test_workspace_sizes():
    d = moe.make_dims(32768, 7168, 3072, 384, 8)
    ffn = moe.ffn_workspace_bytes(d)
    P = 32768 * 8
    # x_q + h_q + per-pair rows (fp16 codes + one scale byte per 32 columns)
    assert ffn >= 32768 * 7168 + P * 3072 + 2 * P * 7168 + P * 7168 // 32
    assert moe.plan_workspace_bytes(d) >= 4 * P
    assert moe.ffn_workspace_bytes(moe.make_dims(4, 200, 512, 8, 2)) == 0   # invalid dims -> 0
    small = moe.make_dims(7, 7168, 3072, 384, 8)
    assert 0 < moe.ffn_workspace_bytes(small) < ffn


def _item_counts(cnt, small_max):
    """Work items of per-expert pair counts, from their definition: experts above
    small_max give one 256-row item per 256 rows (the last one when more than 128
    remain) and one 128-row item for a remainder of 1..128 rows."""
    xl = sum(m // 256 + (m % 256 > 128) for m in cnt if m > small_max)
    large = sum(1 for m in cnt if m > small_max and 1 <= m % 256 <= 128)
    return xl, large


def test_plan_workspace_bounds_hold_and_size_the_layout():
    """The plan workspace is the header and the three item lists, each sized by its
    host-side bound (256-row items: min(P / 129, P / 256 + large experts), since every
    such item holds more than 128 rows), then the planner scratch, every region
    rounded up to 256 bytes. The bounds hold on random and extreme expert sizes."""
    rng = np.random.default_rng(5)
    for T, K, E, sm in [(7, 8, 384, 16), (256, 8, 384, 16), (32768, 8, 384, 16), (300, 1, 1, 16),
                        (2048, 4, 4096, 1), (1000, 8, 64, 40), (129, 1, 1, 16)]:
        P = T * K
        big = min(P // (sm + 1), E)
        xc = min(P // 129, P // 256 + big)
        small = min(P, E) + (P // 16 if sm > 16 else 0)
        nb = max(1, -(-P // 2048))
        al = lambda n: -(-n // 256) * 256
        want = al(64) + al(8 * max(small, 1)) + al(8 * max(big, 1)) + al(8 * max(xc, 1)) + al(4 * max(P, 1))
        want += 2 * al(4 * nb * E)
        assert moe.plan_workspace_bytes(moe.make_dims(T, 256, 256, E, K, small_max=sm)) == want, (T, K, E, sm)
        # random splits of the P pairs over the experts, plus every pair on few experts
        # with 129 rows each (the most 256-row items P pairs can make)
        cases = [np.bincount(rng.integers(0, E, P), minlength=E) for _ in range(20)]
        cases += [np.bincount(rng.zipf(1.3, P) % E, minlength=E)]
        n129 = min(E, P // 129)
        if n129:
            c = np.zeros(E, np.int64)
            c[:n129] = 129
            c[0] += P - 129 * n129
            cases.append(c)
        for cnt in cases:
            assert cnt.sum() == P
            xl, large = _item_counts(cnt.tolist(), sm)
            assert xl <= xc and large <= big, (T, K, E, sm, xl, xc, large, big)


def test_host_checks_reject_before_enqueue():
    L = moe.lib()
    d = moe.make_dims(4, 256, 512, 8, 2)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every check below fails first
    # null outputs
    assert L.moe_plan(ctypes.byref(d), fake, None, fake, fake, fake, fake, 1 << 20, None) == moe.MOE_EINVAL
    # workspace too small
    assert L.moe_plan(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 1, None) == moe.MOE_EWORKSPACE
    args = [fake] * 10
    assert L.moe_ffn(ctypes.byref(d), *args, None, fake, None, fake, 1, None) == moe.MOE_EWORKSPACE
    args[0] = None
    assert L.moe_ffn(ctypes.byref(d), *args, None, fake, None, fake, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(ctypes.byref(d), None, fake, fake, None) == moe.MOE_EINVAL
    # weight packing: an input without its output, and in-place conversion, are refused
    assert L.moe_pack_weights(ctypes.byref(d), fake, None, None, None, None) == moe.MOE_EINVAL
    assert L.moe_pack_weights(ctypes.byref(d), fake, fake, None, None, None) == moe.MOE_EINVAL
    assert L.moe_pack_weights(ctypes.byref(d), None, None, fake, fake, None) == moe.MOE_EINVAL
    bad = moe.make_dims(4, 200, 512, 8, 2)
    assert L.moe_pack_weights(ctypes.byref(bad), fake, ctypes.c_void_p(0x2000), None, None, None) == \
        moe.MOE_EUNSUPPORTED
    assert L.moe_pack_weights(ctypes.byref(d), None, None, None, None, None) == moe.MOE_OK   # nothing to do
    # moe_ffn_static: a call whose workspace exceeds the static scratch is refused on
    # the host, before the scratch is looked up; null arguments as for moe_ffn
    big = moe.make_dims(4096, 1024, 512, 6, 8)
    assert moe.ffn_workspace_bytes(big) > moe.FFN_STATIC_MAX_BYTES
    assert L.moe_ffn_static(ctypes.byref(big), *([fake] * 10), None, fake, None, None) == moe.MOE_ESCRATCH
    assert L.moe_ffn_static(ctypes.byref(big), *([None] * 10), None, fake, None, None) == moe.MOE_EINVAL
    assert "static scratch" in moe.status_string(moe.MOE_ESCRATCH)
    # T == 0 is a no-op for the FFN and the quantizer
    z = moe.make_dims(0, 256, 512, 8, 2)
    assert L.moe_ffn(ctypes.byref(z), *([None] * 10), None, None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_ffn_static(ctypes.byref(z), *([None] * 10), None, None, None, None) == moe.MOE_OK
    assert L.moe_quant_act(ctypes.byref(z), None, None, None, None) == moe.MOE_OK


def test_nvfp4_host_checks():
    """moe_ffn_nvfp4 needs MOE_FLAG_NVFP4 and both tensor-scale arrays; moe_ffn and
    moe_ffn_static refuse NVFP4 dims; all before anything is enqueued."""
    L = moe.lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced
    nv = moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_NVFP4)
    mx = moe.make_dims(4, 256, 512, 8, 2, flags=moe.FLAG_A16)
    ok = [fake] * 13
    assert L.moe_ffn_nvfp4(ctypes.byref(mx), *ok, None, fake, 1 << 30, None) == moe.MOE_EINVAL
    for i in (9, 12):                 # w13_gs, w2_gs
        a = list(ok)
        a[i] = None
        assert L.moe_ffn_nvfp4(ctypes.byref(nv), *a, None, fake, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_ffn_nvfp4(ctypes.byref(nv), *ok, None, fake, 1, None) == moe.MOE_EWORKSPACE
    assert L.moe_ffn_nvfp4(ctypes.byref(nv), *ok, None, None, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_ffn(ctypes.byref(nv), *([fake] * 10), None, fake, None, fake, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_ffn_static(ctypes.byref(nv), *([fake] * 10), None, fake, None, None) == moe.MOE_EINVAL
    z = moe.make_dims(0, 256, 512, 8, 2, flags=moe.FLAG_NVFP4)
    assert L.moe_ffn_nvfp4(ctypes.byref(z), *([None] * 13), None, None, 0, None) == moe.MOE_OK


def test_product_path_has_no_cpu_fallback():
    """The binding raises when the library is absent instead of computing anything."""
    import importlib
    src = open(moe.__file__).read()
    assert "oracle" not in src and "synth" not in src
    assert "raise RuntimeError" in src
    importlib.reload(moe)
