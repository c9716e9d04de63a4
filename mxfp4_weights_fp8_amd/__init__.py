"""Routed MoE FFN with MXFP4 expert weights and online FP8 activations on MI355X.

Thin Python binding over the C-ABI library ``libmoe_mxfp4.so`` (declared in
``include/moe_mxfp4.h``). This module only marshals arguments: torch supplies
device memory and the current HIP stream, every step of the path runs in the
library's HIP kernels. There is no fallback: if the library is missing or a
call fails, an exception is raised.

    plan(topk_ids, E)                     -> Plan          (moe_plan)
    quant_act(x)                          -> (x_q, x_s)    (moe_quant_act)
    ffn(x, topk_weights, plan, weights)   -> y             (moe_ffn)
    ffn(..., static=True)                 -> y             (moe_ffn_static: no workspace)
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
#: workspace bytes moe_ffn_static can serve (MOE_FFN_STATIC_MAX_BYTES)
FFN_STATIC_MAX_BYTES = 64 << 20
EV_START, EV_QUANT_DONE, EV_W13_DONE, EV_W2_DONE, EV_SHARED_DONE, EV_END = range(6)
NUM_EVENTS = 6


class MoEError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("Is", ctypes.c_int32), ("small_max", ctypes.c_int32),
                ("flags", ctypes.c_int32),
                ("tile_w13", ctypes.c_int32), ("tile_w2", ctypes.c_int32)]


#: moe_dims.flags bit: run decode shapes as one persistent W13 -> W2 -> combine launch
FLAG_DECODE_CHAIN = 1
#: moe_dims.flags bit: bf16 activations (MXFP4A16): x not quantized, bf16 SwiGLU rows
FLAG_A16 = 2
#: moe_dims.flags bit: NVFP4 expert weights with bf16 activations (ffn with NVFP4 weights)
FLAG_NVFP4 = 4


class Shared(ctypes.Structure):
    _fields_ = [("w13s", ctypes.c_void_p), ("w13s_s", ctypes.c_void_p), ("w2s", ctypes.c_void_p),
                ("w2s_s", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [("x_q", ctypes.c_void_p), ("x_s", ctypes.c_void_p), ("h_q", ctypes.c_void_p),
                ("h_s", ctypes.c_void_p), ("sh_q", ctypes.c_void_p), ("sh_s", ctypes.c_void_p),
                ("events", ctypes.POINTER(ctypes.c_void_p))]


_lib = None

#: every symbol the header declares, with its ctypes signature
_SIGNATURES = {
    "moe_validate": (ctypes.c_int, [ctypes.POINTER(Dims)]),
    "moe_plan_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "moe_plan": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "moe_quant_act": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 4),
    "moe_pack_weights": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 5),
    "moe_ffn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "moe_ffn": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 10 + [ctypes.POINTER(Shared),
                ctypes.c_void_p, ctypes.POINTER(Debug), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_ffn_static": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 10 + [ctypes.POINTER(Shared),
                       ctypes.c_void_p, ctypes.POINTER(Debug), ctypes.c_void_p]),
    "moe_ffn_nvfp4": (ctypes.c_int, [ctypes.POINTER(Dims)] + [ctypes.c_void_p] * 13 + [ctypes.POINTER(Debug),
                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib() -> ctypes.CDLL:
    """Load the C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_weights_fp8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(code).decode()


def make_dims(T, H, I, E, K, Is=0, small_max=0, flags=0, tile_w13=0, tile_w2=0) -> Dims:
    """moe_dims. tile_w13 / tile_w2: exact-shape tiling per GEMM (0 = the library's
    tuned table, -1 = no 128-row item on the small-M tiles, 1..128 = row limit)."""
    return Dims(int(T), int(H), int(I), int(E), int(K), int(Is), int(small_max), int(flags), int(tile_w13),
                int(tile_w2))


def validate(d: Dims) -> int:
    return lib().moe_validate(ctypes.byref(d))


def plan_workspace_bytes(d: Dims) -> int:
    return lib().moe_plan_workspace_bytes(ctypes.byref(d))


def ffn_workspace_bytes(d: Dims) -> int:
    return lib().moe_ffn_workspace_bytes(ctypes.byref(d))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoEError(rc, what)


def _require(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}")


@dataclasses.dataclass
class Plan:
    dims: Dims
    expert_offsets: torch.Tensor   # [E+1] int32
    sorted_pairs: torch.Tensor     # [P] int32
    pair_rows: torch.Tensor        # [P] int32
    status: torch.Tensor           # [1] int32 (dropped pairs)
    ws: torch.Tensor               # plan workspace (uint8)


def plan(topk_ids: torch.Tensor, E: int, H: int, I: int, small_max: int = 0, Is: int = 0,
         out: Optional[Plan] = None, flags: int = 0, tile_w13: int = 0, tile_w2: int = 0) -> Plan:
    """moe_plan on the current stream. topk_ids: cuda int32 [T, K]. H, I (and Is,
    flags, tile_w13, tile_w2) complete the dims that moe_ffn will use with this plan."""
    T, K = topk_ids.shape
    d = make_dims(T, H, I, E, K, Is, small_max, flags, tile_w13, tile_w2)
    _check(validate(d), "moe_plan dims")
    _require(topk_ids, torch.int32, (T, K), "topk_ids")
    dev = topk_ids.device
    if out is None:
        P = T * K
        out = Plan(d, torch.empty(E + 1, dtype=torch.int32, device=dev),
                   torch.empty(max(P, 1), dtype=torch.int32, device=dev),
                   torch.empty(max(P, 1), dtype=torch.int32, device=dev),
                   torch.zeros(1, dtype=torch.int32, device=dev),
                   torch.empty(plan_workspace_bytes(d), dtype=torch.uint8, device=dev))
    rc = lib().moe_plan(ctypes.byref(d), _ptr(topk_ids), _ptr(out.expert_offsets), _ptr(out.sorted_pairs),
                        _ptr(out.pair_rows), _ptr(out.status), _ptr(out.ws), out.ws.numel(), _stream(dev))
    _check(rc, "moe_plan")
    out.dims = d
    return out


def quant_act(x: torch.Tensor):
    """moe_quant_act: bf16 [T, H] -> (E4M3 codes uint8 [T, H], E8M0 scales uint8 [T, H/128])."""
    T, H = x.shape
    d = make_dims(T, H, 128, 1, 1)
    _check(validate(d), "moe_quant_act dims")
    _require(x, torch.bfloat16, (T, H), "x")
    x_q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    x_s = torch.empty((T, H // 128), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quant_act(ctypes.byref(d), _ptr(x), _ptr(x_q), _ptr(x_s), _stream(x.device)), "moe_quant_act")
    return x_q, x_s


def pack_weights(weights: dict) -> dict:
    """moe_pack_weights on the current stream: a new weights dict whose w13 and w2
    codes are in the kernel-native layout that moe_ffn reads (the scale tensors are
    shared with the input dict). weights: dict w13 [E, 2I, H/2], w13_s, w2
    [E, H, I/2], w2_s (uint8 cuda, row-major codes as produced by MXFP4 packing)."""
    w13, w2 = weights["w13"], weights["w2"]
    E, I2, Hh = w13.shape
    H, I = 2 * Hh, I2 // 2
    _require(w13, torch.uint8, (E, 2 * I, H // 2), "w13")
    _require(w2, torch.uint8, (E, H, I // 2), "w2")
    d = make_dims(1, H, I, E, 1)
    _check(validate(d), "moe_pack_weights dims")
    p13 = torch.empty_like(w13)
    p2 = torch.empty_like(w2)
    _check(lib().moe_pack_weights(ctypes.byref(d), _ptr(w13), _ptr(p13), _ptr(w2), _ptr(p2), _stream(w13.device)),
           "moe_pack_weights")
    out = dict(weights)
    out.update(w13=p13, w2=p2, layout="packed")
    return out


_hip = None


def _hip_rt() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    return _hip


class StageEvents:
    """NUM_EVENTS raw HIP events for moe_ffn's stage boundaries (recorded by the
    library on the stream it launches on)."""

    def __init__(self, only=None):
        """only: optional subset of stage indices to record (the others stay NULL)."""
        h = _hip_rt()
        self.handles = []
        for i in range(NUM_EVENTS):
            e = ctypes.c_void_p()
            if only is None or i in only:
                if h.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
            self.handles.append(e)
        self.array = (ctypes.c_void_p * NUM_EVENTS)(*[e.value for e in self.handles])

    def elapsed_ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        rc = _hip_rt().hipEventElapsedTime(ctypes.byref(out), self.handles[a], self.handles[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def __del__(self):
        try:
            for e in self.handles:
                if e.value:
                    _hip_rt().hipEventDestroy(e)
        except Exception:
            pass


def ffn(x: torch.Tensor, topk_weights: torch.Tensor, p: Plan, weights: dict, shared: Optional[dict] = None,
        debug: bool = False, ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
        events=None, static: bool = False):
    """moe_ffn on the current stream. weights: dict from pack_weights (w13 and w2 in
    the kernel-native layout, w13_s and w2_s row-major; uint8 cuda); shared:
    optional dict w13s, w13s_s, w2s, w2s_s.
    Returns y (bf16 [T, H]); with debug=True returns (y, dict of x_q, x_s, h_q, h_s,
    sh_q, sh_s); with FLAG_A16 or FLAG_NVFP4 in the plan's flags, h_q holds the bf16
    SwiGLU rows (int16 [P, I]) and x_q, x_s, h_s are left as allocated.
    With FLAG_NVFP4 (moe_ffn_nvfp4) the weights dict holds NVFP4 tensors: w13 / w2
    codes (packed), w13_s [E, 2I, H/16] / w2_s [E, H, I/16] E4M3 block scales and
    w13_gs / w2_gs [E] float32 tensor scales. ``events``: optional StageEvents recorded at the stage boundaries.
    ``static``: call moe_ffn_static (the library's static scratch instead of a
    workspace; ``ws`` must then be None)."""
    d = p.dims
    T, H, I, E, K, Is = d.T, d.H, d.I, d.E, d.K, d.Is
    dev = x.device
    _require(x, torch.bfloat16, (T, H), "x")
    _require(topk_weights, torch.float32, (T, K), "topk_weights")
    if weights.get("layout") != "packed":
        raise ValueError("moe_ffn reads expert weights in the kernel-native layout: convert them with pack_weights")
    nv = bool(d.flags & FLAG_NVFP4)
    blk = 16 if nv else 32
    _require(weights["w13"], torch.uint8, (E, 2 * I, H // 2), "w13")
    _require(weights["w13_s"], torch.uint8, (E, 2 * I, H // blk), "w13_s")
    _require(weights["w2"], torch.uint8, (E, H, I // 2), "w2")
    _require(weights["w2_s"], torch.uint8, (E, H, I // blk), "w2_s")
    if nv:
        _require(weights["w13_gs"], torch.float32, (E,), "w13_gs")
        _require(weights["w2_gs"], torch.float32, (E,), "w2_gs")
        if static or (shared is not None and Is > 0):
            raise ValueError("NVFP4 weights run through moe_ffn_nvfp4: no static scratch, no shared expert")
    sh = None
    if shared is not None and Is > 0:
        _require(shared["w13s"], torch.uint8, (2 * Is, H), "w13s")
        _require(shared["w13s_s"], torch.uint8, (2 * Is // 128, H // 128), "w13s_s")
        _require(shared["w2s"], torch.uint8, (H, Is), "w2s")
        _require(shared["w2s_s"], torch.uint8, (H // 128, Is // 128), "w2s_s")
        sh = Shared(shared["w13s"].data_ptr(), shared["w13s_s"].data_ptr(), shared["w2s"].data_ptr(),
                    shared["w2s_s"].data_ptr())
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if static and ws is not None:
        raise ValueError("moe_ffn_static takes no workspace")
    if ws is None and not static:
        ws = torch.empty(ffn_workspace_bytes(d), dtype=torch.uint8, device=dev)
    dbg_t = None
    dbg = None
    ev_arr = None
    if debug or events is not None:
        dbg = Debug()
        if debug:
            P = T * K
            dbg_t = {"x_q": torch.empty((T, H), dtype=torch.uint8, device=dev),
                     "x_s": torch.empty((T, H // 128), dtype=torch.uint8, device=dev),
                     "h_q": torch.zeros((max(P, 1), I),
                                        dtype=torch.int16 if d.flags & (FLAG_A16 | FLAG_NVFP4) else torch.uint8,
                                        device=dev),
                     "h_s": torch.zeros((max(P, 1), I // 128), dtype=torch.uint8, device=dev),
                     "sh_q": torch.zeros((T, max(Is, 128)), dtype=torch.uint8, device=dev),
                     "sh_s": torch.zeros((T, max(Is, 128) // 128), dtype=torch.uint8, device=dev)}
            for k, v in dbg_t.items():
                setattr(dbg, k, v.data_ptr())
        if events is not None:
            ev_arr = events.array
            dbg.events = ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p))
    args = [ctypes.byref(d), _ptr(x), _ptr(topk_weights), _ptr(p.expert_offsets), _ptr(p.sorted_pairs),
            _ptr(p.pair_rows), _ptr(p.ws), _ptr(weights["w13"]), _ptr(weights["w13_s"]), _ptr(weights["w2"]),
            _ptr(weights["w2_s"]), ctypes.byref(sh) if sh is not None else None, _ptr(y),
            ctypes.byref(dbg) if dbg is not None else None]
    if nv:
        _check(lib().moe_ffn_nvfp4(ctypes.byref(d), _ptr(x), _ptr(topk_weights), _ptr(p.expert_offsets),
                                   _ptr(p.sorted_pairs), _ptr(p.pair_rows), _ptr(p.ws), _ptr(weights["w13"]),
                                   _ptr(weights["w13_s"]), _ptr(weights["w13_gs"]), _ptr(weights["w2"]),
                                   _ptr(weights["w2_s"]), _ptr(weights["w2_gs"]), _ptr(y),
                                   ctypes.byref(dbg) if dbg is not None else None, _ptr(ws), ws.numel(),
                                   _stream(dev)), "moe_ffn_nvfp4")
    elif static:
        _check(lib().moe_ffn_static(*args, _stream(dev)), "moe_ffn_static")
    else:
        _check(lib().moe_ffn(*args, _ptr(ws), ws.numel(), _stream(dev)), "moe_ffn")
    if debug:
        return y, dbg_t
    return y
