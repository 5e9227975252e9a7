"""Packed low-bit weight-only GEMV / verify GEMM for MI355X (gfx950).

Thin Python binding of ``libqgemv.so`` (C ABI in ``include/qgemv.h``): it only
marshals arguments -- device pointers of PyTorch tensors and the current HIP
stream -- into the library, where every step of the computation runs in HIP
kernels.  PyTorch is used for device memory and streams only.  There is no CPU
fallback: if the library is not built, or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

__all__ = ["QGError", "lib", "QLinear", "mlp", "run_batch", "stream_read", "declared_symbols", "LIB_PATH",
           "HEADER_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qgemv.h")

QG_OK, QG_ERR_INVALID_ARG, QG_ERR_UNSUPPORTED, QG_ERR_DEVICE, QG_ERR_OOM = 0, -1, -2, -3, -4
FMT_UNIFORM, FMT_TRELLIS3, FMT_MXFP4, FMT_MXFP6 = 0, 1, 2, 3
FLAG_X_PREROTATED = 1
FLAG_BATCH_INVARIANT = 2
GROUP = 128
# pins (include/qgemv.h): force a kernel or hand-over
PIN_M1_PERGROUP, PIN_M1_RUNS, PIN_PARTIALS, PIN_WORDS = 1 << 0, 1 << 1, 1 << 2, 1 << 3
PIN_XS_T1, PIN_XS_T2, PIN_TRELLIS_ROT_LAUNCH, PIN_TRELLIS_BAND = 1 << 4, 1 << 5, 1 << 6, 1 << 7


class QGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"qgemv status {status}: {msg}")
        self.status = status


class _Launch(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_int32), ("waves", ctypes.c_int32), ("splits", ctypes.c_int32)]


class _Desc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("format", ctypes.c_int32), ("bits", ctypes.c_int32), ("col_bits", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("codebook", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("pins", ctypes.c_uint32), ("launch", _Launch * 3)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqgemv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                          f"python bit_weight_only_packed_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u16p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    L.qgemv_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(_Desc), i32, vp]
    L.qgemv_run.argtypes = [vp, vp, i32, vp, vp]
    L.qmlp_run.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    L.qgemv_destroy.argtypes = [vp]
    L.qg_last_error.argtypes = []
    L.qg_last_error.restype = ctypes.c_char_p
    L.qgemv_weight_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_int64)]
    L.qg_stream_read.argtypes = [vp, ctypes.c_int64, vp]
    L.qgemv_run_batch.argtypes = [i32, vp, vp, vp, i32, vp]
    L.qgemv_run_noalloc.argtypes = [vp, vp, i32, vp, vp]
    L.qgemv_debug_unpack.argtypes = [vp, vp, vp]
    L.qgemv_debug_dequant.argtypes = [vp, vp, u16p, vp]
    L.qgemv_debug_operand.argtypes = [vp, vp, vp, vp, vp]
    L.qgemv_debug_trellis.argtypes = [vp, vp, vp]
    L.qgemv_run_prefill.argtypes = [vp, vp, i32, vp, vp, ctypes.c_size_t, vp]
    L.qgemv_prefill_workspace.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    for f in ("qgemv_create", "qgemv_run", "qmlp_run", "qgemv_destroy", "qgemv_weight_bytes", "qg_stream_read",
              "qgemv_run_batch", "qgemv_run_noalloc", "qgemv_run_prefill", "qgemv_prefill_workspace",
              "qgemv_debug_unpack", "qgemv_debug_dequant", "qgemv_debug_operand", "qgemv_debug_trellis"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def declared_symbols() -> list:
    """Function names declared in include/qgemv.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+)\s*\(", text)))


def _check(st: int):
    if st != QG_OK:
        raise QGError(st, lib().qg_last_error().decode(errors="replace"))


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t) -> int:
    return int(t.data_ptr())


class QLinear:
    """One packed weight matrix W[N][K] held by a library handle.

    codes: CUDA tensor holding the canonical packed stream (uniform: uint32
    words, any 4-byte dtype; trellis: uint16 words [N/16][K/16][48], any 2-byte
    dtype).  scales: CUDA fp16 tensor [N][K/128].  bits: 2/3/4, or col_bits
    (host array of per-column widths).  codebook: CUDA fp16 [65536] (trellis).
    pins: PIN_* bits; launch: optional {row class 0/1/2: (tiles, waves, splits)}
    launch-geometry overrides (both fixed at create).  batch_invariant: row m of
    an M-row run is bit-identical to running that row alone (uniform codes).
    group_size: the scale group, 128 (scales [N][K/128]) or, for uniform
    codes, 64 or 32 (scales [N][K/64] or [N][K/32]).  mxfp4: codes are E2M1
    elements in the 4-bit stream, scales a CUDA uint8 tensor of UE8M0 bytes
    [N][K/32].  mxfp6: codes are E3M2 elements in the 6-bit stream, scales as
    for mxfp4.
    """

    def __init__(self, codes, scales, K: int, N: int, bits: int = 3, col_bits=None, max_M: int = 32,
                 trellis: bool = False, codebook=None, prerotated: bool = False, stream=None,
                 pins: int = 0, launch=None, batch_invariant: bool = False, group_size: int = GROUP,
                 mxfp4: bool = False, mxfp6: bool = False):
        d = _Desc()
        mx = mxfp4 or mxfp6
        d.K, d.N, d.group_size = int(K), int(N), 32 if mx else int(group_size)
        d.format = FMT_TRELLIS3 if trellis else (FMT_MXFP4 if mxfp4 else (FMT_MXFP6 if mxfp6 else FMT_UNIFORM))
        self._cb_host = None
        if not trellis and col_bits is not None:
            self._cb_host = np.ascontiguousarray(np.asarray(col_bits, dtype=np.uint8))
            d.bits = 0
            d.col_bits = self._cb_host.ctypes.data
        else:
            d.bits = 0 if trellis else (4 if mxfp4 else (6 if mxfp6 else int(bits)))
        d.codes = _ptr(codes)
        d.scales = _ptr(scales)
        d.codebook = _ptr(codebook) if codebook is not None else None
        d.flags = (FLAG_X_PREROTATED if prerotated else 0) | (FLAG_BATCH_INVARIANT if batch_invariant else 0)
        d.pins = int(pins)
        for c, (t, w, s) in (launch or {}).items():
            d.launch[int(c)] = _Launch(int(t), int(w), int(s))
        h = ctypes.c_void_p()
        _check(lib().qgemv_create(ctypes.byref(h), ctypes.byref(d), int(max_M), _stream(stream)))
        self._h = h
        self.K, self.N, self.max_M, self.trellis = int(K), int(N), int(max_M), trellis

    @property
    def handle(self):
        return self._h

    def run(self, x, out=None, stream=None):
        import torch
        M = x.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        _check(lib().qgemv_run(self._h, _ptr(x), int(M), _ptr(out), _stream(stream)))
        return out

    __call__ = run

    def prefill_workspace(self):
        """(least, full) workspace bytes of run_prefill."""
        lo, full = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().qgemv_prefill_workspace(self._h, ctypes.byref(lo), ctypes.byref(full)))
        return int(lo.value), int(full.value)

    def run_prefill(self, x, out=None, workspace=None, stream=None):
        """y = x W^T for any row count through the dequantise-then-fp16-GEMM route.
        workspace: a CUDA uint8 tensor (default: the full size, allocated here)."""
        import torch
        M = x.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        if workspace is None:
            workspace = torch.empty(self.prefill_workspace()[1], dtype=torch.uint8, device=x.device)
        nbytes = int(workspace.numel() * workspace.element_size())
        _check(lib().qgemv_run_prefill(self._h, _ptr(x), int(M), _ptr(out), _ptr(workspace), nbytes, _stream(stream)))
        return out

    def weight_bytes(self) -> int:
        b = ctypes.c_int64()
        _check(lib().qgemv_weight_bytes(self._h, ctypes.byref(b)))
        return int(b.value)

    def debug_unpack(self, stream=None):
        import torch
        c = torch.full((self.N, self.K), -1, dtype=torch.int32, device="cuda")
        _check(lib().qgemv_debug_unpack(self._h, _ptr(c), _stream(stream)))
        return c

    def debug_dequant(self, with_q16: bool = True, stream=None):
        import torch
        w = torch.full((self.N, self.K), float("nan"), dtype=torch.float32, device="cuda")
        q = torch.zeros((self.N, self.K), dtype=torch.float16, device="cuda") if with_q16 else None
        _check(lib().qgemv_debug_dequant(self._h, _ptr(w), _ptr(q) if q is not None else None, _stream(stream)))
        return w, q

    def debug_operand(self, stream=None):
        """The verify GEMM's operand decode: (codes int32, operand fp16 bits, w fp32), all [N][K]."""
        import torch
        c = torch.full((self.N, self.K), -1, dtype=torch.int32, device="cuda")
        b = torch.zeros((self.N, self.K), dtype=torch.int16, device="cuda")
        w = torch.full((self.N, self.K), float("nan"), dtype=torch.float32, device="cuda")
        _check(lib().qgemv_debug_operand(self._h, _ptr(c), _ptr(b), _ptr(w), _stream(stream)))
        return c, b, w

    def debug_trellis(self, stream=None):
        import torch
        s = torch.zeros((self.N, self.K), dtype=torch.int16, device="cuda")
        _check(lib().qgemv_debug_trellis(self._h, _ptr(s), _stream(stream)))
        return s

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().qgemv_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def run_batch(lins, xs, outs=None, stream=None):
    """Several independent products y_i = x_i W_i^T (same row count) in one call
    (one launch at M = 1).  lins: QLinear list; xs: CUDA fp16 tensors [M][K_i]."""
    import torch
    n = len(lins)
    M = xs[0].shape[0]
    if outs is None:
        outs = [torch.empty((M, l.N), dtype=torch.float16, device=x.device) for l, x in zip(lins, xs)]
    H = (ctypes.c_void_p * n)(*[l.handle.value for l in lins])
    X = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    Y = (ctypes.c_void_p * n)(*[_ptr(y) for y in outs])
    _check(lib().qgemv_run_batch(n, H, X, Y, int(M), _stream(stream)))
    return outs


def stream_read(buf, stream=None):
    """Plain streaming read of a CUDA tensor's bytes (the measured read roofline)."""
    _check(lib().qg_stream_read(_ptr(buf), int(buf.numel() * buf.element_size()), _stream(stream)))


def mlp(gate: QLinear, up: QLinear, down: QLinear, x, out=None, stream=None):
    """out = down(SiLU(gate(x)) * up(x)) in two fused launches."""
    import torch
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, down.N), dtype=torch.float16, device=x.device)
    _check(lib().qmlp_run(gate.handle, up.handle, down.handle, _ptr(x), int(M), _ptr(out), _stream(stream)))
    return out
