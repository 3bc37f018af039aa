"""Thin ctypes binding of libda2 (the C ABI in include/da2.h).

Argument marshalling only: every step of the hot path runs in the HIP
library.  PyTorch supplies device memory (tensors) and streams.  Importing
this module raises if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libda2.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "da2.h")

DBG = {name: i for i, name in enumerate([
    "Q_I8", "Q_I8_SCALE", "Q_MX", "Q_MX_SCALE", "K_I8", "K_I8_SCALE", "K_MX", "K_MX_SCALE",
    "V_FP8", "V_FP8_SCALE", "V_MX", "V_MX_SCALE", "Q_AVG", "K_AVG", "Q_MAX", "K_MAX", "KEYS",
    "SCHEDULE"])}


class Da2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))
        self.status = status


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("frames", C.c_int32), ("height", C.c_int32), ("width", C.c_int32),
                ("stride_b", C.c_int64), ("stride_h", C.c_int64), ("stride_n", C.c_int64),
                ("prefix", C.c_int32), ("capacity", C.c_int32)]


class Budget(C.Structure):
    _fields_ = [("hi_bp", C.c_int32), ("lo_bp", C.c_int32), ("lambda_", C.c_double),
                ("scope", C.c_int32), ("full_bp", C.c_int32), ("skip_means", C.c_int32)]


_lib = None


def lib():
    """Load libda2.so; raise when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libda2.so is not built (python -m video_diffusion_dit_frame_amd.build)")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.da2_layout_create.argtypes = [C.POINTER(Shape), C.POINTER(P)]
        L.da2_layout_destroy.argtypes = [P]
        L.da2_layout_regions.argtypes = [P, C.POINTER(i32)]
        L.da2_layout_regions.restype = i32
        L.da2_layout_slots.argtypes = [P, P]
        L.da2_layout_slots.restype = C.c_int
        L.da2_workspace_bytes.argtypes = [P]
        L.da2_workspace_bytes.restype = sz
        L.da2_plan_create.argtypes = [P, P, sz, C.POINTER(P)]
        L.da2_plan_destroy.argtypes = [P]
        L.da2_plan.argtypes = [P, P, P, C.POINTER(Budget), P]
        L.da2_plan_from_tier_map.argtypes = [P, P, P, P, P]
        L.da2_plan_tier_map.argtypes = [P, P, P]
        L.da2_attention.argtypes = [P, P, P, P, P, i32, P]
        L.da2_attention_prefixed.argtypes = [P, P, P, P, P, P, P, P, P, P, i32, P]
        L.da2_plan_debug.argtypes = [P, i32, P, P]
        L.da2_plan_debug_bytes.argtypes = [P, i32]
        L.da2_plan_debug_bytes.restype = sz
        L.da2_status_string.argtypes = [C.c_int]
        L.da2_status_string.restype = C.c_char_p
        L.da2_exp_constants.argtypes = [P]
        L.da2_plan_timing.argtypes = [P, i32]
        L.da2_plan_timing.restype = C.c_int
        L.da2_plan_timing_read.argtypes = [P, P, i32, C.POINTER(i32)]
        L.da2_plan_timing_read.restype = C.c_int
        L.da2_quotas.argtypes = [i64, i32, i32, i32, C.POINTER(i64), C.POINTER(i64), C.POINTER(i64)]
        L.da2_forward_noalloc.argtypes = [P, P, P, P, P, C.POINTER(Budget), i32, P]
        for name in ("da2_layout_create", "da2_plan_create", "da2_plan", "da2_plan_from_tier_map",
                     "da2_plan_tier_map", "da2_attention", "da2_attention_prefixed",
                     "da2_plan_debug", "da2_forward_noalloc"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def header_functions():
    """Names of the functions include/da2.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(da2_[a-z_]+)\s*\(", text)))


def _out_dtype(o) -> int:
    if o.dtype == torch.float32:
        return 1
    if o.dtype == torch.bfloat16:
        return 0
    raise TypeError("output must be float32 or bfloat16")


def status_string(st: int) -> str:
    return lib().da2_status_string(int(st)).decode()


def _check(st: int, what: str):
    if st != 0:
        raise Da2Error(st, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def exp_constants():
    import numpy as np

    out = np.empty(17, np.float64)
    lib().da2_exp_constants(out.ctypes.data_as(C.c_void_p))
    return out


def quotas3(n, full_bp, hi_bp, lo_bp):
    """Cumulative quotas (T16, T16 + T8, T16 + T8 + T4) for n pairs."""
    t16, t8, tk = C.c_int64(), C.c_int64(), C.c_int64()
    lib().da2_quotas(int(n), int(full_bp), int(hi_bp), int(lo_bp), C.byref(t16), C.byref(t8),
                     C.byref(tk))
    return t16.value, t8.value, tk.value


def quotas(n, hi_bp, lo_bp):
    """(T8, T8 + T4) with no 16-bit share."""
    _, t8, tk = quotas3(n, 0, hi_bp, lo_bp)
    return t8, tk


class Layout:
    """Region layout for one shape.  q/k/v/o are addressed with the given
    element strides (channel stride 1).  cap: block capacity (64 or 128);
    R regions (Rf per frame) of cap slots, T = R cap / 64 tiles."""

    def __init__(self, B, H, d, F, Hv, Wv, stride_b, stride_h, stride_n, prefix=0, cap=64):
        self.B, self.H, self.d, self.F, self.Hv, self.Wv = B, H, d, F, Hv, Wv
        self.N = F * Hv * Wv
        self.prefix = prefix
        self.cap = cap
        self.shape = Shape(B, H, d, F, Hv, Wv, stride_b, stride_h, stride_n, prefix, cap)
        h = C.c_void_p()
        _check(lib().da2_layout_create(C.byref(self.shape), C.byref(h)), "da2_layout_create")
        self.handle = h
        rf = C.c_int32()
        self.R = int(lib().da2_layout_regions(h, C.byref(rf)))
        self.Rf = rf.value
        self.Np = cap * self.R
        self.T = self.Np // 64

    def slots(self):
        """One frame's partition: int32 [R_f, cap], token y*Wv + x of each slot
        (-1: padding)."""
        import numpy as np

        out = np.empty((self.Rf, self.cap), np.int32)
        _check(lib().da2_layout_slots(self.handle, out.ctypes.data_as(C.c_void_p)), "da2_layout_slots")
        return out

    @classmethod
    def for_tensor(cls, x: torch.Tensor, F, Hv, Wv, bhnd=True, prefix=0, cap=64):
        """x: a [B, H, N, d] view (bhnd) or a [B, N, H, d] view, channel-contiguous."""
        if bhnd:
            B, H, N, d = x.shape
            sb, sh, sn, sc = x.stride()
        else:
            B, N, H, d = x.shape
            sb, sn, sh, sc = x.stride()
        assert sc == 1 and N == F * Hv * Wv
        return cls(B, H, d, F, Hv, Wv, sb, sh, sn, prefix, cap)

    @property
    def workspace_bytes(self) -> int:
        return int(lib().da2_workspace_bytes(self.handle))

    def debug_bytes(self, which) -> int:
        return int(lib().da2_plan_debug_bytes(self.handle, DBG[which] if isinstance(which, str) else which))

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.da2_layout_destroy(self.handle)
            self.handle = None


class Plan:
    """A plan bound to a caller-owned device workspace."""

    def __init__(self, layout: Layout, workspace: torch.Tensor = None):
        self.layout = layout
        if workspace is None:
            workspace = torch.empty(layout.workspace_bytes, dtype=torch.uint8, device="cuda")
        self.workspace = workspace
        h = C.c_void_p()
        _check(lib().da2_plan_create(layout.handle, C.c_void_p(workspace.data_ptr()),
                                     workspace.numel() * workspace.element_size(), C.byref(h)),
               "da2_plan_create")
        self.handle = h

    def plan(self, q, k, hi_bp, lo_bp, lam=0.2, scope=0, stream=None, full_bp=0, skip_means=False):
        b = Budget(int(hi_bp), int(lo_bp), float(lam), int(scope), int(full_bp), int(bool(skip_means)))
        _check(lib().da2_plan(self.handle, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                              C.byref(b), _stream(stream)), "da2_plan")

    def plan_from_tier_map(self, q, k, tier: torch.Tensor, stream=None):
        assert tier.dtype == torch.uint8 and tier.is_contiguous()
        L = self.layout
        assert tier.numel() == L.B * L.H * L.R * L.R
        _check(lib().da2_plan_from_tier_map(self.handle, C.c_void_p(q.data_ptr()),
                                            C.c_void_p(k.data_ptr()), C.c_void_p(tier.data_ptr()),
                                            _stream(stream)), "da2_plan_from_tier_map")

    def tier_map(self, stream=None) -> torch.Tensor:
        L = self.layout
        out = torch.empty((L.B, L.H, L.R, L.R), dtype=torch.uint8, device="cuda")
        _check(lib().da2_plan_tier_map(self.handle, C.c_void_p(out.data_ptr()), _stream(stream)),
               "da2_plan_tier_map")
        return out

    def attention(self, q, k, v, o, stream=None):
        _check(lib().da2_attention(self.handle, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                                   C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), _out_dtype(o),
                                   _stream(stream)), "da2_attention")

    def attention_prefixed(self, q, k, v, o, qp, kp, vp, op, valid=None, stream=None):
        """Joint text-video attention: video q/k/v/o plus the text prefix
        qp/kp/vp/op ([B,H,Lp,d] views with the video strides); valid: device
        int32 [B] valid prefix keys, or None for all."""
        assert op.dtype == o.dtype
        if valid is not None:
            assert valid.dtype == torch.int32 and valid.is_cuda and valid.numel() == self.layout.B
        ptr = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        _check(lib().da2_attention_prefixed(self.handle, ptr(q), ptr(k), ptr(v), ptr(o), ptr(qp), ptr(kp),
                                            ptr(vp), ptr(op), ptr(valid), _out_dtype(o), _stream(stream)),
               "da2_attention_prefixed")

    def debug(self, which, stream=None) -> torch.Tensor:
        w = DBG[which] if isinstance(which, str) else int(which)
        n = self.layout.debug_bytes(w)
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
        _check(lib().da2_plan_debug(self.handle, w, C.c_void_p(out.data_ptr()), _stream(stream)),
               "da2_plan_debug")
        return out

    def timing(self, enable: bool):
        """Record HIP events around the attention kernel of later calls."""
        _check(lib().da2_plan_timing(self.handle, int(bool(enable))), "da2_plan_timing")

    def timing_read(self):
        """Per-call attention-kernel durations (ms) recorded since timing(True)."""
        import numpy as np

        n = C.c_int32()
        _check(lib().da2_plan_timing_read(self.handle, None, 0, C.byref(n)), "da2_plan_timing_read")
        out = np.empty(max(n.value, 1), np.float32)
        _check(lib().da2_plan_timing_read(self.handle, out.ctypes.data_as(C.c_void_p), n.value,
                                          C.byref(n)), "da2_plan_timing_read")
        return out[:n.value]

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.da2_plan_destroy(self.handle)
            self.handle = None


def noalloc_bytes() -> int:
    """DA2_NOALLOC_BYTES of include/da2.h: the library's own workspace per GPU."""
    with open(HEADER) as f:
        m = re.search(r"#define DA2_NOALLOC_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    return int(m.group(1)) << int(m.group(2))


def forward_noalloc(layout: Layout, q, k, v, o, hi_bp, lo_bp, lam=0.2, scope=0, stream=None, full_bp=0,
                    skip_means=False):
    """da2_forward_noalloc: plan + attention on the library's own workspace
    (for callers that cannot allocate device memory)."""
    b = Budget(int(hi_bp), int(lo_bp), float(lam), int(scope), int(full_bp), int(bool(skip_means)))
    _check(lib().da2_forward_noalloc(layout.handle, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                                     C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), C.byref(b),
                                     _out_dtype(o), _stream(stream)), "da2_forward_noalloc")


def to_device_bf16(x_u16, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bits (numpy) -> bfloat16 device tensor, same shape."""
    import numpy as np

    t = torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16))
    return t.view(torch.bfloat16).to(device)
