"""Fused 4-bit + low-rank-adapter linear layer for AMD MI355X (gfx950).

Thin Python binding over ``libqlin.so`` (C ABI in ``include/qlin.h``).  The
functions keep the C names; torch is used only to own device memory and to
supply the current HIP stream.  Every step of the computation runs in the
library's HIP kernels; when the library is missing the calls raise.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np

from ._lib import (EXPORTS, LIB_PATH, QLIN_FMT_INT4_GROUP, QLIN_FMT_NF, QLIN_FMT_NF4, QlinError,
                   QWeightStruct, check, lib)

__all__ = [
    "QWeight", "QlinError", "qlin_nf4_codebook", "qlin_quantize_nf4", "qlin_nf_codebook",
    "qlin_quantize_nf",
    "qlin_quantize_int4_group", "qlin_workspace_bytes", "qlin_fwd", "qlin_fwd_noalloc", "qlin_bwd",
    "qlin_dequant_bf16", "qlin_qa_merge", "qlin_int4_scale_zero_grad", "qlin_profile_next_launch", "EXPORTS", "LIB_PATH",
]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} CUDA tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} "
                         f"cuda={t.is_cuda}")


@dataclasses.dataclass
class QWeight:
    """A packed frozen weight and the tensors that own its device memory."""
    format: int
    block: int
    dq_block: int
    d_out: int
    d_in: int
    codes: object                 # uint8 [d_out][d_in/2]
    absmax: object = None         # NF4: int8 [n_blocks] (dq) or float32 [n_blocks]
    absmax2: object = None        # NF4 dq: float32 [ceil(n_blocks/dq_block)]
    scale: object = None          # INT4: fp16 [d_out][d_in/group]
    zero: object = None
    bits: int = 0                 # NF: 2, 3 or 4

    def struct(self) -> QWeightStruct:
        return QWeightStruct(self.format, self.block, self.dq_block, self.bits, self.d_out, self.d_in,
                             _ptr(self.codes), _ptr(self.absmax), _ptr(self.absmax2),
                             _ptr(self.scale), _ptr(self.zero))

    @property
    def device(self):
        return self.codes.device

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.codes, self.absmax, self.absmax2, self.scale, self.zero) if t is not None)


def qlin_nf4_codebook() -> np.ndarray:
    out = (ctypes.c_float * 16)()
    check(lib().qlin_nf4_codebook(out), "qlin_nf4_codebook")
    return np.frombuffer(out, dtype=np.float32).copy()


def qlin_quantize_nf4(W, block: int = 64, dq_block: int = 256) -> QWeight:
    torch = _torch()
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W")
    nb = d_out * d_in // block if block > 0 else 0
    dev = W.device
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    if dq_block:
        absmax = torch.empty(nb, dtype=torch.int8, device=dev)
        absmax2 = torch.empty(-(-nb // dq_block), dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
        absmax2 = None
    check(lib().qlin_quantize_nf4(W.data_ptr(), d_out, d_in, block, dq_block, codes.data_ptr(),
                                  absmax.data_ptr(), _ptr(absmax2), _stream(dev)),
          "qlin_quantize_nf4")
    return QWeight(QLIN_FMT_NF4, block, dq_block, d_out, d_in, codes, absmax, absmax2)


def qlin_lq_nf4(W, r: int, iters: int, power: int, omega_t, dq_block: int = 256):
    """Low-rank plus quantized decomposition W ~ Q + B A (Q NF4 with blocks of
    64; B [d_out][r] and A [r][d_in] bf16, for the layer with s = 1).
    omega_t: fp32 [r][d_in] start of the subspace iteration (drawn by the
    caller).  Returns (QWeight, B, A, errs) with errs[t] the relative
    reconstruction error after iteration t."""
    torch = _torch()
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W")
    dev = W.device
    if r > 0:
        _need(omega_t, torch.float32, (r, d_in), "omega_t")
    nb = d_out * d_in // 64
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    if dq_block:
        absmax = torch.empty(nb, dtype=torch.int8, device=dev)
        absmax2 = torch.empty(-(-nb // dq_block), dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
        absmax2 = None
    B = torch.empty((d_out, max(r, 1)), dtype=torch.bfloat16, device=dev)[:, :r]
    A = torch.empty((max(r, 1), d_in), dtype=torch.bfloat16, device=dev)[:r]
    errs = torch.empty(iters, dtype=torch.float32, device=dev)
    nbytes = lib().qlin_lq_workspace_bytes(d_out, d_in, r)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    check(lib().qlin_lq_nf4(W.data_ptr(), d_out, d_in, r, iters, power,
                            omega_t.data_ptr() if r > 0 else None, dq_block, codes.data_ptr(),
                            absmax.data_ptr(), _ptr(absmax2), B.data_ptr() if r > 0 else None,
                            A.data_ptr() if r > 0 else None, errs.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream(dev)), "qlin_lq_nf4")
    return QWeight(QLIN_FMT_NF4, 64, dq_block, d_out, d_in, codes, absmax, absmax2), B, A, errs


def qlin_nf_codebook(bits: int) -> np.ndarray:
    out = (ctypes.c_float * 16)()
    check(lib().qlin_nf_codebook(bits, out), "qlin_nf_codebook")
    return np.frombuffer(out, dtype=np.float32)[: 1 << bits].copy()


def qlin_quantize_nf(W, bits: int, block: int, dq_block: int = 256) -> QWeight:
    torch = _torch()
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W")
    nb = d_out * d_in // block
    dev = W.device
    codes = torch.empty((d_out, d_in * bits // 8), dtype=torch.uint8, device=dev)
    if dq_block:
        absmax = torch.empty(nb, dtype=torch.int8, device=dev)
        absmax2 = torch.empty(-(-nb // dq_block), dtype=torch.float32, device=dev)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
        absmax2 = None
    check(lib().qlin_quantize_nf(W.data_ptr(), d_out, d_in, bits, block, dq_block, codes.data_ptr(),
                                 absmax.data_ptr(), _ptr(absmax2), _stream(dev)), "qlin_quantize_nf")
    return QWeight(QLIN_FMT_NF, block, dq_block, d_out, d_in, codes, absmax, absmax2, bits=bits)


def qlin_quantize_int4_group(W, group: int = 32) -> QWeight:
    torch = _torch()
    d_out, d_in = W.shape
    _need(W, torch.float32, (d_out, d_in), "W")
    dev = W.device
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    scale = torch.empty((d_out, d_in // group), dtype=torch.float16, device=dev)
    zero = torch.empty((d_out, d_in // group), dtype=torch.float16, device=dev)
    check(lib().qlin_quantize_int4_group(W.data_ptr(), d_out, d_in, group, codes.data_ptr(),
                                         scale.data_ptr(), zero.data_ptr(), _stream(dev)),
          "qlin_quantize_int4_group")
    return QWeight(QLIN_FMT_INT4_GROUP, group, 0, d_out, d_in, codes, scale=scale, zero=zero)


def qlin_workspace_bytes(w: QWeight, M: int, r: int, pool: int = 1) -> int:
    s = w.struct()
    n = lib().qlin_workspace_bytes(ctypes.byref(s), M, r, pool)
    if n == 0:
        raise QlinError(2, "qlin_workspace_bytes")
    return n


_WS = {}


def workspace(device, nbytes: int):
    """A zero-filled per-device workspace of at least ``nbytes`` (grown on demand).
    Calls on one stream may share it; calls in flight on different streams may not."""
    torch = _torch()
    key = str(device)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def qlin_fwd(w: QWeight, x, A, B, r: int, s: float, pool: int = 1, y=None, u_out=None,
             ws=None, want_u: bool = True):
    """y = x W_bf16^T + s (P A^T) B^T.  Returns (y, u) (u is None unless wanted).
    r = 0 is the layer without an adapter (A and B may be None; no u)."""
    torch = _torch()
    M = x.shape[0]
    dev = x.device
    _need(x, torch.bfloat16, (M, w.d_in), "x")
    if r > 0:
        _need(A, torch.bfloat16, (r, w.d_in // pool), "A")
        _need(B, torch.bfloat16, (w.d_out, r), "B")
    else:
        want_u = False
    if y is None:
        y = torch.empty((M, w.d_out), dtype=torch.bfloat16, device=dev)
    if u_out is None and want_u:
        u_out = torch.empty((M, r), dtype=torch.float32, device=dev)
    nbytes = qlin_workspace_bytes(w, M, r, pool)
    if ws is None:
        ws = workspace(dev, nbytes)
    s_ = w.struct()
    check(lib().qlin_fwd(ctypes.byref(s_), x.data_ptr(), M, _ptr(A), _ptr(B), r,
                         float(s), pool, y.data_ptr(), _ptr(u_out), ws.data_ptr(), ws.numel(),
                         _stream(dev)), "qlin_fwd")
    return y, u_out


def qlin_fwd_noalloc(w: QWeight, x, A, B, r: int, s: float, pool: int = 1, y=None, u_out=None,
                     want_u: bool = True):
    """qlin_fwd without a workspace (the library's own device array; see
    include/qlin.h).  Output tensors are allocated here unless passed in."""
    torch = _torch()
    M = x.shape[0]
    dev = x.device
    _need(x, torch.bfloat16, (M, w.d_in), "x")
    if r > 0:
        _need(A, torch.bfloat16, (r, w.d_in // pool), "A")
        _need(B, torch.bfloat16, (w.d_out, r), "B")
    else:
        want_u = False
    if y is None:
        y = torch.empty((M, w.d_out), dtype=torch.bfloat16, device=dev)
    if u_out is None and want_u:
        u_out = torch.empty((M, r), dtype=torch.float32, device=dev)
    s_ = w.struct()
    check(lib().qlin_fwd_noalloc(ctypes.byref(s_), x.data_ptr(), M, _ptr(A), _ptr(B), r, float(s),
                                 pool, y.data_ptr(), _ptr(u_out), _stream(dev)), "qlin_fwd_noalloc")
    return y, u_out


def qlin_bwd(w: QWeight, x, A, B, r: int, s: float, dy, pool: int = 1, u_saved=None,
             need_dx: bool = True, dx=None, dA=None, dB=None, ws=None):
    """Returns (dx, dA, dB): dX = dY W_bf16 + expand(du A), dA = du^T P, dB = s dY^T u."""
    torch = _torch()
    M = x.shape[0]
    dev = x.device
    _need(x, torch.bfloat16, (M, w.d_in), "x")
    _need(dy, torch.bfloat16, (M, w.d_out), "dy")
    if need_dx and dx is None:
        dx = torch.empty((M, w.d_in), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((r, w.d_in // pool), dtype=torch.bfloat16, device=dev)
    if dB is None:
        dB = torch.empty((w.d_out, r), dtype=torch.bfloat16, device=dev)
    nbytes = qlin_workspace_bytes(w, M, r, pool)
    if ws is None:
        ws = workspace(dev, nbytes)
    s_ = w.struct()
    check(lib().qlin_bwd(ctypes.byref(s_), x.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                         float(s), pool, dy.data_ptr(), _ptr(u_saved),
                         _ptr(dx) if need_dx else None, dA.data_ptr(), dB.data_ptr(),
                         ws.data_ptr(), ws.numel(), _stream(dev)), "qlin_bwd")
    return dx, dA, dB


def qlin_qa_merge(w: QWeight, A, B, r: int, s: float, zero_out=None):
    """Merged fp16 zero points RN16(zero + s B A) of an INT4 weight; returns
    a new QWeight sharing codes and scales with ``w`` and holding them."""
    torch = _torch()
    G = w.d_in // w.block
    _need(A, torch.bfloat16, (r, G), "A")
    _need(B, torch.bfloat16, (w.d_out, r), "B")
    if zero_out is None:
        zero_out = torch.empty((w.d_out, G), dtype=torch.float16, device=w.device)
    s_ = w.struct()
    check(lib().qlin_qa_merge(ctypes.byref(s_), A.data_ptr(), B.data_ptr(), r, float(s),
                              zero_out.data_ptr(), _stream(w.device)), "qlin_qa_merge")
    return dataclasses.replace(w, zero=zero_out)


def qlin_int4_scale_zero_grad(w: QWeight, x, dy, dscale=None, dzero=None):
    """fp32 gradients (dscale, dzero) [d_out][d_in/32] of an INT4 weight's
    group scales and zero points."""
    torch = _torch()
    M = x.shape[0]
    dev = x.device
    G = w.d_in // w.block
    _need(x, torch.bfloat16, (M, w.d_in), "x")
    _need(dy, torch.bfloat16, (M, w.d_out), "dy")
    if dscale is None:
        dscale = torch.empty((w.d_out, G), dtype=torch.float32, device=dev)
    if dzero is None:
        dzero = torch.empty((w.d_out, G), dtype=torch.float32, device=dev)
    s_ = w.struct()
    check(lib().qlin_int4_scale_zero_grad(ctypes.byref(s_), x.data_ptr(), M, dy.data_ptr(),
                                          dscale.data_ptr(), dzero.data_ptr(), _stream(dev)),
          "qlin_int4_scale_zero_grad")
    return dscale, dzero


def qlin_dequant_bf16(w: QWeight):
    torch = _torch()
    out = torch.empty((w.d_out, w.d_in), dtype=torch.bfloat16, device=w.device)
    s_ = w.struct()
    check(lib().qlin_dequant_bf16(ctypes.byref(s_), out.data_ptr(), _stream(w.device)),
          "qlin_dequant_bf16")
    return out


def qlin_profile_next_launch(kernel: Optional[str], start=None, stop=None) -> None:
    """Record torch.cuda.Event ``start`` / ``stop`` around the next launch of
    ``kernel`` (None disarms).  The events must already exist on the device
    (record each once before arming)."""
    if kernel is None:
        check(lib().qlin_profile_next_launch(None, None, None), "qlin_profile_next_launch")
        return
    check(lib().qlin_profile_next_launch(kernel.encode(), start.cuda_event, stop.cuda_event),
          "qlin_profile_next_launch")
