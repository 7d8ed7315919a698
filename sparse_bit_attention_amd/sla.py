"""ctypes binding of libsagesla (argument marshalling only).

Every step of the forward runs in the HIP kernels behind ``include/sagesla.h``;
PyTorch only supplies device memory and the stream.  Importing this module
raises if the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsagesla.so")

SLA_OK, SLA_EINVAL, SLA_EUNSUPPORTED, SLA_EWORKSPACE, SLA_EHIP, SLA_ENOMEM, SLA_ETOOLARGE = range(7)
NOALLOC_WS_BYTES = 64 << 20  # SLA_NOALLOC_WS_BYTES
WS_REGIONS = ["QBAR", "KSUM", "KBAR", "MU", "MASK", "KEPT", "Q8", "K8", "DQ", "DK", "LSE"]

EXPORTS = ["sla_plan", "sla_plan_destroy", "sla_plan_info", "sla_quantize", "sla_attention_fwd",
           "sla_prepare_kv", "sla_attend", "sla_status_string", "sla_ws_view",
           "sla_debug_qk_int32", "sla_quant_b128", "sla_w8a8_gemm", "sla_attention_bwd",
           "sla_attention_fwd_noalloc"]


class SlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class sla_config(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("block", ctypes.c_int32), ("topk", ctypes.c_float),
                ("use_linear", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("qk_int8", ctypes.c_int32), ("qk_fine", ctypes.c_int32),
                ("backward", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_bit_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.sla_plan.argtypes = [ctypes.POINTER(sla_config), ctypes.POINTER(P)]
        L.sla_plan.restype = ctypes.c_int
        L.sla_plan_destroy.argtypes = [P]
        L.sla_plan_destroy.restype = ctypes.c_int
        L.sla_plan_info.argtypes = [P, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(sz)]
        L.sla_plan_info.restype = ctypes.c_int
        L.sla_quantize.argtypes = [P, P, P, P, sz, P]
        L.sla_quantize.restype = ctypes.c_int
        L.sla_attention_fwd.argtypes = [P, P, P, P, P, P, P, sz, P]
        L.sla_attention_fwd.restype = ctypes.c_int
        L.sla_prepare_kv.argtypes = [P, P, P, P, P, sz, P]
        L.sla_prepare_kv.restype = ctypes.c_int
        L.sla_attend.argtypes = [P, P, P, P, sz, P]
        L.sla_attend.restype = ctypes.c_int
        L.sla_status_string.argtypes = [ctypes.c_int]
        L.sla_status_string.restype = ctypes.c_char_p
        L.sla_ws_view.argtypes = [P, P, i32, ctypes.POINTER(P), ctypes.POINTER(sz)]
        L.sla_ws_view.restype = ctypes.c_int
        L.sla_debug_qk_int32.argtypes = [P, P, P, i32, P, P]
        L.sla_debug_qk_int32.restype = ctypes.c_int
        L.sla_quant_b128.argtypes = [P, i32, i32, P, P, P]
        L.sla_quant_b128.restype = ctypes.c_int
        L.sla_w8a8_gemm.argtypes = [P, P, P, P, i32, i32, i32, P, P]
        L.sla_w8a8_gemm.restype = ctypes.c_int
        L.sla_attention_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.sla_attention_bwd.restype = ctypes.c_int
        L.sla_attention_fwd_noalloc.argtypes = [P, P, P, P, P, P, P]
        L.sla_attention_fwd_noalloc.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().sla_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != SLA_OK:
        raise SlaError(status, where)


@dataclass
class PlanInfo:
    T: int
    kb: int
    workspace_bytes: int


class Plan:
    """Owns an ``sla_plan_t``."""

    def __init__(self, B, H, N, d, topk, use_linear=True, sm_scale=0.0, qk_int8=True, block=64,
                 qk_fine=False, backward=False):
        self.cfg = sla_config(B, H, N, d, block, topk, int(use_linear), sm_scale, int(qk_int8),
                              int(qk_fine), int(backward))
        h = ctypes.c_void_p()
        _check(lib().sla_plan(ctypes.byref(self.cfg), ctypes.byref(h)), "sla_plan")
        self.handle = h
        T, kb, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
        _check(lib().sla_plan_info(h, ctypes.byref(T), ctypes.byref(kb), ctypes.byref(ws)),
               "sla_plan_info")
        self.info = PlanInfo(T.value, kb.value, ws.value)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.sla_plan_destroy(h)
            self.handle = None

    def ws_region(self, ws_ptr: int, which: str):
        p, n = ctypes.c_void_p(), ctypes.c_size_t()
        _check(lib().sla_ws_view(self.handle, ctypes.c_void_p(ws_ptr), WS_REGIONS.index(which),
                                 ctypes.byref(p), ctypes.byref(n)), "sla_ws_view")
        return (p.value or 0) - ws_ptr, n.value


class SageSLA:
    """SageSLA forward (and, for plain SLA with backward=True, its backward) on
    [B, H, N, d] bf16 CUDA (HIP) tensors."""

    def __init__(self, B, H, N, d, topk, use_linear=True, sm_scale=0.0, qk_int8=True,
                 device="cuda", qk_fine=False, backward=False):
        import torch
        self.plan = Plan(B, H, N, d, topk, use_linear, sm_scale, qk_int8, qk_fine=qk_fine,
                         backward=backward)
        self.qk_fine = bool(qk_fine)
        self.shape = (B, H, N, d)
        self.use_linear = bool(use_linear)
        self.device = torch.device(device)
        self.ws = torch.empty(max(self.plan.info.workspace_bytes, 256), dtype=torch.uint8,
                              device=self.device)

    # -- helpers ---------------------------------------------------------------
    def _tensor(self, x, name, shape):
        import torch
        if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
        return ctypes.c_void_p(x.data_ptr())

    @staticmethod
    def _stream(stream):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        return ctypes.c_void_p(s.cuda_stream)

    # -- the two calls ---------------------------------------------------------
    def quantize(self, q, k, stream=None):
        _check(lib().sla_quantize(self.plan.handle, self._tensor(q, "q", self.shape),
                                  self._tensor(k, "k", self.shape),
                                  ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                  self._stream(stream)), "sla_quantize")

    def attention(self, q, k, v, w=None, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(self.shape, dtype=torch.bfloat16, device=self.device)
        d = self.shape[3]
        wp = self._tensor(w, "w", (d, d)) if w is not None else ctypes.c_void_p(0)
        _check(lib().sla_attention_fwd(self.plan.handle, self._tensor(q, "q", self.shape),
                                       self._tensor(k, "k", self.shape),
                                       self._tensor(v, "v", self.shape), wp,
                                       self._tensor(out, "out", self.shape),
                                       ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                       self._stream(stream)), "sla_attention_fwd")
        return out

    def prepare_kv(self, k, v, w=None, stream=None):
        d = self.shape[3]
        wp = self._tensor(w, "w", (d, d)) if w is not None else ctypes.c_void_p(0)
        _check(lib().sla_prepare_kv(self.plan.handle, self._tensor(k, "k", self.shape),
                                    self._tensor(v, "v", self.shape), wp,
                                    ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                    self._stream(stream)), "sla_prepare_kv")

    def attend(self, q, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(self.shape, dtype=torch.bfloat16, device=self.device)
        _check(lib().sla_attend(self.plan.handle, self._tensor(q, "q", self.shape),
                                self._tensor(out, "out", self.shape),
                                ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                self._stream(stream)), "sla_attend")
        return out

    def forward(self, q, k, v, w=None, out=None, stream=None):
        self.quantize(q, k, stream)
        return self.attention(q, k, v, w, out, stream)

    __call__ = forward

    def backward(self, q, k, v, w, dout, dq=None, dk=None, dv=None, dw=None, stream=None):
        """Gradients (dq, dk, dv bf16 [B,H,N,d]; dw float32 [d,d] or None) of
        sum(dout * out) after forward() on the same inputs (plain SLA)."""
        import torch
        d = self.shape[3]

        def new(x):
            return x if x is not None else torch.empty(self.shape, dtype=torch.bfloat16,
                                                       device=self.device)
        dq, dk, dv = new(dq), new(dk), new(dv)
        if self.use_linear and dw is None:
            dw = torch.empty((d, d), dtype=torch.float32, device=self.device)
        if dw is not None and (dw.dtype != torch.float32 or tuple(dw.shape) != (d, d)
                               or not dw.is_contiguous()):
            raise ValueError("dw must be a contiguous float32 [d, d] device tensor")
        wp = self._tensor(w, "w", (d, d)) if w is not None else ctypes.c_void_p(0)
        _check(lib().sla_attention_bwd(
            self.plan.handle, self._tensor(q, "q", self.shape), self._tensor(k, "k", self.shape),
            self._tensor(v, "v", self.shape), wp, self._tensor(dout, "dout", self.shape), self._tensor(dq, "dq", self.shape),
            self._tensor(dk, "dk", self.shape), self._tensor(dv, "dv", self.shape),
            ctypes.c_void_p(dw.data_ptr() if dw is not None else 0),
            ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(), self._stream(stream)),
            "sla_attention_bwd")
        return dq, dk, dv, dw

    # -- debug views -----------------------------------------------------------
    def region(self, which: str):
        """A torch view of one workspace region (see sagesla.h)."""
        import torch
        off, n = self.plan.ws_region(self.ws.data_ptr(), which)
        raw = self.ws[off:off + n]
        B, H, N, d = self.shape
        T, kb = self.plan.info.T, self.plan.info.kb
        BH = B * H
        if which in ("QBAR", "KSUM", "KBAR"):
            return raw.view(torch.float32).view(BH, T, d)
        if which == "MU":
            return raw.view(torch.float32).view(BH, d)
        if which in ("DQ", "DK"):
            if self.qk_fine:  # one scale per 16 query rows / per 4 keys
                return raw.view(torch.float32).view(BH, T, 4 if which == "DQ" else 16)
            return raw.view(torch.float32).view(BH, T)
        if which == "MASK":
            return raw.view(torch.int64).view(BH, T, (T + 63) // 64)
        if which == "KEPT":
            return raw.view(torch.int32).view(BH, T, max(kb, 1))[:, :, :kb]
        if which in ("Q8", "K8"):
            return raw.view(torch.int8).view(BH, T, 64 * d)
        if which == "LSE":
            return raw.view(torch.float32).view(BH, T, 64)
        raise KeyError(which)

    def debug_qk_int32(self, triples, stream=None):
        """int32 QK^T tiles [n, 64, 64] for (bh, i, j) triples."""
        import torch
        t = torch.as_tensor(triples, dtype=torch.int32).reshape(-1, 3).contiguous().to(self.device)
        n = t.shape[0]
        out = torch.empty((n, 64, 64), dtype=torch.int32, device=self.device)
        _check(lib().sla_debug_qk_int32(self.plan.handle, ctypes.c_void_p(self.ws.data_ptr()),
                                        ctypes.c_void_p(t.data_ptr()), n,
                                        ctypes.c_void_p(out.data_ptr()), self._stream(stream)),
               "sla_debug_qk_int32")
        return out


def i8_unswizzle(tiles, d):
    """Fragment-ordered INT8 blocks [..., 64*d] -> row-major [..., 64, d]
    (pure index permutation, layout documented in sagesla.h)."""
    import numpy as np
    r = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    KC = d // 64
    off = ((((r >> 4) * KC + (c >> 6)) * 64 + (r & 15) + 16 * ((c & 63) >> 4)) << 4) + (c & 15)
    return np.asarray(tiles)[..., off]


# ---- W8A8 linear layers (see sagesla.h) ----------------------------------------

def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def quant_b128(x, stream=None):
    """bf16 [R, C] (cuda) -> (int8 codes [R, C], float32 scales [ceil(R/128), ceil(C/128)])."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    R, C = x.shape
    codes = torch.empty((R, C), dtype=torch.int8, device=x.device)
    scales = torch.empty(((R + 127) // 128, (C + 127) // 128), dtype=torch.float32, device=x.device)
    _check(lib().sla_quant_b128(ctypes.c_void_p(x.data_ptr()), R, C,
                                ctypes.c_void_p(codes.data_ptr()),
                                ctypes.c_void_p(scales.data_ptr()), _stream_handle(stream)),
           "sla_quant_b128")
    return codes, scales


def w8a8_gemm(xq, sx, wq, sw, out=None, stream=None):
    """Block-scaled INT8 GEMM: bf16 [M, N] = dequant(xq) dequant(wq)^T."""
    import torch
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and xq.dtype == torch.int8 and wq.dtype == torch.int8
    assert xq.is_contiguous() and wq.is_contiguous() and sx.is_contiguous() and sw.is_contiguous()
    assert sx.shape == ((M + 127) // 128, K // 128) and sw.shape == ((N + 127) // 128, K // 128)
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(lib().sla_w8a8_gemm(ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sx.data_ptr()),
                               ctypes.c_void_p(wq.data_ptr()), ctypes.c_void_p(sw.data_ptr()),
                               M, N, K, ctypes.c_void_p(y.data_ptr()), _stream_handle(stream)),
           "sla_w8a8_gemm")
    return y


def attention_fwd_noalloc(plan: Plan, q, k, v, w, out, stream=None):
    """sla_attention_fwd_noalloc: the forward (quantisation included) on the
    library's static per-GPU workspace.  q, k, v, out: contiguous bf16
    [B,H,N,d] device tensors of the plan's shape; w: bf16 [d,d] or None.
    Allocates nothing."""
    import torch
    B, H, N, d = plan.cfg.B, plan.cfg.H, plan.cfg.N, plan.cfg.d
    for name, x, shape in (("q", q, (B, H, N, d)), ("k", k, (B, H, N, d)), ("v", v, (B, H, N, d)),
                           ("out", out, (B, H, N, d))) + ((("w", w, (d, d)),) if w is not None else ()):
        if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
        if tuple(x.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {shape}")
    s = stream if stream is not None else torch.cuda.current_stream()
    ptr = lambda x: ctypes.c_void_p(x.data_ptr() if x is not None else 0)
    _check(lib().sla_attention_fwd_noalloc(plan.handle, ptr(q), ptr(k), ptr(v), ptr(w), ptr(out),
                                           ctypes.c_void_p(s.cuda_stream)),
           "sla_attention_fwd_noalloc")
    return out
