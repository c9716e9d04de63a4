"""Lane images for single-MFMA tests (test support; no method arithmetic).

Builds the per-lane register images that tests/native/mfma_probe.hip feeds to
one MFMA instruction, from logical matrices of element codes, and reads the
16 x 16 result back. Lane layouts, gfx950, lane l, q = l // 16:

v_mfma_scale_f32_16x16x128_f8f6f4 (A 16 x 128, B 128 x 16):
  A: row l % 16; B: column l % 16.
  8-bit operand: bytes 0..15 hold K = 16q + i, bytes 16..31 hold K = 64 + 16q + i.
  4-bit operand: bytes 0..15 hold K = 32q .. 32q + 31, low nibble first.
  scale operand: byte 0 = E8M0 of row / column l % 16 for K block q (32q .. 32q+31).
v_mfma_f32_16x16x32_bf16 (A 16 x 32, B 32 x 16): bf16 K = 8q .. 8q + 7.
Both: D (and C) lane l holds column l % 16, rows 4q .. 4q + 3.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

E4M3, E2M1 = 0, 4
HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "native", "libmfma_probe.so")


def _lane_bytes_8bit(m16x128: np.ndarray) -> np.ndarray:
    """[16, 128] codes (row = lane % 16) -> [64, 32] bytes."""
    out = np.zeros((64, 32), dtype=np.uint8)
    for l in range(64):
        q, r = l // 16, l % 16
        out[l, :16] = m16x128[r, 16 * q:16 * q + 16]
        out[l, 16:] = m16x128[r, 64 + 16 * q:64 + 16 * q + 16]
    return out


def _lane_bytes_4bit(m16x128: np.ndarray) -> np.ndarray:
    out = np.zeros((64, 32), dtype=np.uint8)
    for l in range(64):
        q, r = l // 16, l % 16
        k = m16x128[r, 32 * q:32 * q + 32].astype(np.uint8)
        out[l, :16] = (k[0::2] & 0xF) | ((k[1::2] & 0xF) << 4)
    return out


def scaled_images(a_codes, b_codes, a_scales, b_scales, fmt_a, fmt_b, c=None):
    """a_codes [16, 128] (row, K), b_codes [128, 16] (K, column) element codes;
    a_scales [16, 4], b_scales [16, 4] (row or column, K block) E8M0 codes;
    c [16, 16] float32 or None. Returns (a, b, sa, sb, c) lane images."""
    pa = _lane_bytes_4bit if fmt_a == E2M1 else _lane_bytes_8bit
    pb = _lane_bytes_4bit if fmt_b == E2M1 else _lane_bytes_8bit
    a = pa(np.asarray(a_codes)).view(np.int32).reshape(64, 8)
    b = pb(np.asarray(b_codes).T.copy()).view(np.int32).reshape(64, 8)
    lanes = np.arange(64)
    sa = np.asarray(a_scales, dtype=np.int32)[lanes % 16, lanes // 16]
    sb = np.asarray(b_scales, dtype=np.int32)[lanes % 16, lanes // 16]
    return a, b, sa, sb, c_image(c)


def bf16_images(a_bits, b_bits, c=None):
    """a_bits [16, 32] (row, K), b_bits [32, 16] (K, column) bf16 bit patterns."""
    a16 = np.zeros((64, 16), dtype=np.uint16)
    b16 = np.zeros((64, 16), dtype=np.uint16)
    A = np.asarray(a_bits, dtype=np.uint16)
    B = np.asarray(b_bits, dtype=np.uint16)
    for l in range(64):
        q, r = l // 16, l % 16
        a16[l, :8] = A[r, 8 * q:8 * q + 8]
        b16[l, :8] = B[8 * q:8 * q + 8, r]
    return a16.view(np.int32).reshape(64, 8), b16.view(np.int32).reshape(64, 8), c_image(c)


def c_image(c) -> np.ndarray:
    out = np.zeros((64, 4), dtype=np.float32)
    if c is None:
        return out
    c = np.asarray(c, dtype=np.float32)
    for l in range(64):
        q, col = l // 16, l % 16
        out[l] = c[4 * q:4 * q + 4, col]
    return out


def d_matrix(d_lanes: np.ndarray) -> np.ndarray:
    """[64, 4] float32 lane image -> [16, 16] (row, column)."""
    out = np.zeros((16, 16), dtype=np.float32)
    for l in range(64):
        q, col = l // 16, l % 16
        out[4 * q:4 * q + 4, col] = d_lanes[l]
    return out


_lib = None


def probe_lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(PROBE_LIB)
        L.probe_mfma_scaled.restype = ctypes.c_int
        L.probe_mfma_scaled.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6 + [ctypes.c_int,
                                                                                              ctypes.c_void_p]
        L.probe_mfma_bf16.restype = ctypes.c_int
        L.probe_mfma_bf16.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
        L.probe_cvt_fp4_bf16.restype = ctypes.c_int
        L.probe_cvt_fp4_bf16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
        L.probe_cvt_fp4_f32.restype = ctypes.c_int
        L.probe_cvt_fp4_f32.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


def run_scaled(cases, fmt_a, fmt_b, device="cuda:0"):
    """cases: list of (a, b, sa, sb, c) lane images -> list of [16, 16] results."""
    import torch
    n = len(cases)
    A = torch.from_numpy(np.stack([x[0] for x in cases])).to(device)
    B = torch.from_numpy(np.stack([x[1] for x in cases])).to(device)
    SA = torch.from_numpy(np.stack([x[2] for x in cases]).astype(np.int32)).to(device)
    SB = torch.from_numpy(np.stack([x[3] for x in cases]).astype(np.int32)).to(device)
    C = torch.from_numpy(np.stack([x[4] for x in cases])).to(device)
    D = torch.zeros_like(C)
    s = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    rc = probe_lib().probe_mfma_scaled(fmt_a, fmt_b, A.data_ptr(), B.data_ptr(), SA.data_ptr(), SB.data_ptr(),
                                       C.data_ptr(), D.data_ptr(), n, s)
    assert rc == 0, rc
    torch.cuda.synchronize()
    Dn = D.cpu().numpy()
    return [d_matrix(Dn[i]) for i in range(n)]


def run_bf16(cases, device="cuda:0"):
    import torch
    n = len(cases)
    A = torch.from_numpy(np.stack([x[0] for x in cases])).to(device)
    B = torch.from_numpy(np.stack([x[1] for x in cases])).to(device)
    C = torch.from_numpy(np.stack([x[2] for x in cases])).to(device)
    D = torch.zeros_like(C)
    s = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    rc = probe_lib().probe_mfma_bf16(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), n, s)
    assert rc == 0, rc
    torch.cuda.synchronize()
    Dn = D.cpu().numpy()
    return [d_matrix(Dn[i]) for i in range(n)]
