"""Python binding of ``libmoe_ffn_fp8.so`` (the C ABI in ``include/moe_ffn_fp8.h``).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU; the binding passes their
``data_ptr()`` and the current HIP stream.  There is no fallback: if the library is
missing, :func:`load` raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_FFN_FP8_LIB names another build of the same library (a variant
# made with `python -m fp8_moe_ffn_amd.build --out PATH ...`)
LIB_PATH = os.environ.get("MOE_FFN_FP8_LIB") or os.path.join(_PKG, "libmoe_ffn_fp8.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_OUT_OF_MEMORY = -3
ERR_HIP = -4
NUM_STAGES = 3
CHUNK = 16  # tokens per kernel launch (MOE_FFN_FP8_CHUNK)
SCRATCH_BYTES = 8 << 20  # the allocation-free forward's static scratch per device (MOE_FFN_FP8_SCRATCH_BYTES)
GROUP_MAX = 1024  # tokens per grouped pass (MOE_FFN_FP8_GROUP_MAX)
GROUP_FROM = 8  # batches above this many tokens run grouped (MOE_FFN_FP8_GROUP_FROM)
BATCH_GROUPED = 0  # batches above GROUP_FROM tokens: grouped passes (the default)
BATCH_CHUNKED = 1  # batches above GROUP_FROM tokens: launches of up to CHUNK tokens
LAUNCH_THREE = 0   # a launch of the decode kernels: three kernels (the default)
LAUNCH_SINGLE = 1  # the same as one kernel in three phases (hidden 5120, up to 8 tokens)
STAGE_NAMES = ("fc13_swiglu", "fc2", "combine")

# Every function declared in include/moe_ffn_fp8.h: name -> (restype, argtypes)
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "moe_ffn_fp8_create": (_i32, [_vp, _vp]),
    "moe_ffn_fp8_prepack_expert": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_fp8_prepack": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_fp8_unpack_expert": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_fp8_forward": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp]),
    "moe_ffn_fp8_forward_scratch": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp]),
    "moe_ffn_fp8_forward_debug": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "moe_ffn_fp8_forward_variant": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_ffn_fp8_forward_rmsnorm": (_i32, [_vp, _vp, ctypes.c_float, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_ffn_fp8_set_batch_mode": (_i32, [_vp, _i32]),
    "moe_ffn_fp8_set_launch_mode": (_i32, [_vp, _i32]),
    "moe_ffn_fp8_profile_begin": (_i32, [_vp]),
    "moe_ffn_fp8_profile_end": (_i32, [_vp, _vp, _vp]),
    "moe_ffn_fp8_destroy": (_i32, [_vp]),
    "moe_ffn_fp8_status_string": (ctypes.c_char_p, [_i32]),
    "moe_ffn_fp8_e4m3_encode": (_i32, [_vp, _vp, _i64, _vp]),
    "moe_ffn_fp8_e4m3_decode": (_i32, [_vp, _vp, _i64, _vp]),
    "moe_ffn_fp8_e4m3_quantize": (_i32, [_vp, ctypes.c_float, _vp, _i64, _vp]),
    "moe_ffn_fp8_stream_read": (_i32, [_vp, _i64, _vp, _vp]),
}

_lib = None


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("max_tokens", ctypes.c_int32)]


class DebugPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("xq", "s_x", "expert", "gate", "aq_shared", "s_a_shared", "aq_routed",
                 "s_a_routed", "num_active", "sync_timeouts")]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the shared library (once) and declare every exported signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m fp8_moe_ffn_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().moe_ffn_fp8_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise MoeError(status, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Variant(ctypes.Structure):
    """moe_ffn_fp8_variant: the variant readings (all zero: the step as built)."""

    _fields_ = [("gate_on_input", ctypes.c_int32), ("x_scale", ctypes.c_float), ("a_scale", ctypes.c_float)]


@dataclass
class DebugOut:
    xq: object
    s_x: object
    expert: object
    gate: object
    aq_shared: object
    s_a_shared: object
    aq_routed: object
    s_a_routed: object
    num_active: object
    sync_timeouts: object


class MoeFFN:
    """One handle: packed weights of E routed experts plus the shared expert."""

    def __init__(self, hidden: int, inter: int, num_experts: int, max_tokens: int):
        lib = load()
        self.dims = Dims(hidden, inter, num_experts, max_tokens)
        h = ctypes.c_void_p()
        _check(lib.moe_ffn_fp8_create(ctypes.byref(self.dims), ctypes.byref(h)), "create")
        self._h = h

    @classmethod
    def prepacked(cls, hidden: int, inter: int, num_experts: int, max_tokens: int, w13, w2, s13, s2,
                  stream=None) -> "MoeFFN":
        """A handle made by moe_ffn_fp8_prepack from stacked device tensors: w13 uint8
        [E+1][K][2I], w2 uint8 [E+1][I][K], s13 float32 [E+1][2I], s2 float32 [E+1][K]."""
        self = cls.__new__(cls)
        self.dims = Dims(hidden, inter, num_experts, max_tokens)
        h = ctypes.c_void_p()
        _check(load().moe_ffn_fp8_prepack(ctypes.byref(self.dims), _ptr(w13), _ptr(w2), _ptr(s13), _ptr(s2),
                                          _stream(stream), ctypes.byref(h)), "prepack")
        self._h = h
        return self

    @property
    def handle(self) -> int:
        return self._h.value

    def prepack_expert(self, slot: int, w13, s13, w2, s2, stream=None):
        """slot 0..E-1 routed, E shared; uint8 / float32 device tensors."""
        _check(load().moe_ffn_fp8_prepack_expert(self._h, slot, _ptr(w13), _ptr(s13), _ptr(w2),
                                                 _ptr(s2), _stream(stream)), "prepack_expert")

    def unpack_expert(self, slot: int, w13, s13, w2, s2, stream=None):
        _check(load().moe_ffn_fp8_unpack_expert(self._h, slot, _ptr(w13), _ptr(s13), _ptr(w2),
                                                _ptr(s2), _stream(stream)), "unpack_expert")

    def forward(self, x, logits, out, stream=None):
        """x, out: bf16 [M][K]; logits: bf16 [M][E] or None (dense)."""
        _check(load().moe_ffn_fp8_forward(_ptr(x), _ptr(logits), self._h, _ptr(out),
                                          x.shape[0], _stream(stream)), "forward")
        return out

    def forward_scratch(self, x, logits, out, stream=None):
        """The allocation-free forward (the library's static scratch instead of the handle's
        workspace; at most min(max_tokens, CHUNK) tokens)."""
        _check(load().moe_ffn_fp8_forward_scratch(_ptr(x), _ptr(logits), self._h, _ptr(out),
                                                  x.shape[0], _stream(stream)), "forward_scratch")
        return out

    def forward_raw(self, x_ptr, logits_ptr, out_ptr, m: int, stream_handle) -> int:
        """Pointer-level call (for timing loops); returns the status."""
        return load().moe_ffn_fp8_forward(x_ptr, logits_ptr, self._h, out_ptr, m, stream_handle)

    def forward_debug(self, x, logits, out, dbg: DebugOut, stream=None):
        ptrs = DebugPtrs(*(_ptr(getattr(dbg, f)) for f, _ in DebugPtrs._fields_))
        _check(load().moe_ffn_fp8_forward_debug(_ptr(x), _ptr(logits), self._h, _ptr(out),
                                                x.shape[0], _stream(stream), ctypes.byref(ptrs)),
               "forward_debug")
        return out

    def forward_variant(self, x, logits, out, variant: "Variant", dbg: "DebugOut" = None, stream=None):
        ptrs = (ctypes.byref(DebugPtrs(*(_ptr(getattr(dbg, f)) for f, _ in DebugPtrs._fields_)))
                if dbg is not None else None)
        _check(load().moe_ffn_fp8_forward_variant(_ptr(x), _ptr(logits), self._h, _ptr(out), x.shape[0],
                                                  _stream(stream), ctypes.byref(variant), ptrs),
               "forward_variant")
        return out

    def forward_rmsnorm(self, h, norm_w, eps: float, logits, out, variant: "Variant" = None,
                        dbg: "DebugOut" = None, stream=None):
        """The step on rmsnorm(h) * norm_w, the norm fused into the first kernel."""
        ptrs = (ctypes.byref(DebugPtrs(*(_ptr(getattr(dbg, f)) for f, _ in DebugPtrs._fields_)))
                if dbg is not None else None)
        _check(load().moe_ffn_fp8_forward_rmsnorm(_ptr(h), _ptr(norm_w), ctypes.c_float(eps), _ptr(logits),
                                                  self._h, _ptr(out), h.shape[0], _stream(stream),
                                                  ctypes.byref(variant) if variant is not None else None, ptrs),
               "forward_rmsnorm")
        return out

    def forward_rmsnorm_raw(self, h_ptr, norm_w_ptr, eps: float, logits_ptr, out_ptr, m: int, stream_handle,
                            variant: "Variant" = None) -> int:
        return load().moe_ffn_fp8_forward_rmsnorm(h_ptr, norm_w_ptr, ctypes.c_float(eps), logits_ptr, self._h,
                                                  out_ptr, m, stream_handle,
                                                  ctypes.byref(variant) if variant is not None else None, None)

    def forward_variant_raw(self, x_ptr, logits_ptr, out_ptr, m: int, stream_handle, variant: "Variant") -> int:
        return load().moe_ffn_fp8_forward_variant(x_ptr, logits_ptr, self._h, out_ptr, m, stream_handle,
                                                  ctypes.byref(variant), None)

    def set_batch_mode(self, mode: int):
        """BATCH_GROUPED or BATCH_CHUNKED: how a forward above GROUP_FROM tokens runs."""
        _check(load().moe_ffn_fp8_set_batch_mode(self._h, mode), "set_batch_mode")

    def set_launch_mode(self, mode: int):
        """LAUNCH_THREE or LAUNCH_SINGLE: how a launch of the decode kernels is enqueued."""
        _check(load().moe_ffn_fp8_set_launch_mode(self._h, mode), "set_launch_mode")

    def profile_begin(self):
        _check(load().moe_ffn_fp8_profile_begin(self._h), "profile_begin")

    def profile_end(self):
        """-> (list of summed ms per stage, number of forwards recorded)."""
        ms = (ctypes.c_float * NUM_STAGES)()
        calls = ctypes.c_int32()
        _check(load().moe_ffn_fp8_profile_end(self._h, ms, ctypes.byref(calls)), "profile_end")
        return list(ms), calls.value

    def close(self):
        if self._h is not None and self._h.value:
            _check(load().moe_ffn_fp8_destroy(self._h), "destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def debug_buffers(m: int, hidden: int, inter: int, device="cuda") -> DebugOut:
    import torch

    z = lambda *s, dt: torch.zeros(*s, dtype=dt, device=device)
    return DebugOut(
        xq=z(m, hidden, dt=torch.uint8), s_x=z(m, dt=torch.float32),
        expert=z(m, dt=torch.int32), gate=z(m, dt=torch.float32),
        aq_shared=z(m, inter, dt=torch.uint8), s_a_shared=z(m, dt=torch.float32),
        aq_routed=z(m, inter, dt=torch.uint8), s_a_routed=z(m, dt=torch.float32),
        num_active=z(1, dt=torch.int32), sync_timeouts=z(1, dt=torch.int32))


def e4m3_encode(values, stream=None):
    import torch

    out = torch.empty(values.shape, dtype=torch.uint8, device=values.device)
    _check(load().moe_ffn_fp8_e4m3_encode(_ptr(values), _ptr(out), values.numel(), _stream(stream)),
           "e4m3_encode")
    return out


def e4m3_quantize(values, scale: float, stream=None):
    """Codes of values / scale (float32 device tensor, host scale > 0)."""
    import torch

    out = torch.empty(values.shape, dtype=torch.uint8, device=values.device)
    _check(load().moe_ffn_fp8_e4m3_quantize(_ptr(values), ctypes.c_float(scale), _ptr(out), values.numel(),
                                            _stream(stream)), "e4m3_quantize")
    return out


def stream_read(buf, sink, stream=None):
    """Enqueue the streaming-read probe over a device tensor (its bytes; sink: a device
    tensor of at least 4 bytes)."""
    _check(load().moe_ffn_fp8_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                          _stream(stream)), "stream_read")


def e4m3_decode(codes, stream=None):
    import torch

    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(load().moe_ffn_fp8_e4m3_decode(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)),
           "e4m3_decode")
    return out


def build_from_experts(experts: Sequence, num_experts: int, max_tokens: int, stream=None) -> MoeFFN:
    """Create a handle and prepack ``experts[slot]`` (objects with w13, s13, w2, s2 device
    tensors) for slots 0..E (slot E is the shared expert)."""
    e0 = experts[0]
    hidden, two_i = e0.w13.shape
    m = MoeFFN(hidden, two_i // 2, num_experts, max_tokens)
    for slot in range(num_experts + 1):
        e = experts[slot]
        m.prepack_expert(slot, e.w13, e.s13, e.w2, e.s2, stream)
    return m
