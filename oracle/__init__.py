"""CPU oracle for INT8 conv_fprop (INT32 output, or a requantising INT8
epilogue) — test infrastructure only.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg use this
package.  The product path never imports it.  It wraps the plain nested-loop C
implementation in ``conv_fprop_oracle.c`` (64-bit sums over the definition on
the cuDNN "Convolutions" page, section "Convolution Fprop"; loop order and
strided addressing from "Building a From-Scratch INT8 Strided Convolution
Kernel", steps 1 and 2) through ctypes, marshalling torch CPU tensors (any
strides) into pointers, dims and element strides.

Parity status: every entry point here is pinned by ``tests/test_oracle_pins.py``
(brute force, a float64 library convolution, closed forms, invariants and
mutation checks), none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

from . import build as _build

__all__ = ["OracleError", "Oracle", "load", "out_dims", "conv_fprop", "conv_fprop_points",
           "conv_fprop_requant", "requant_values", "conv_dgrad", "conv_wgrad", "max_threads"]

_ERRORS = {
    1: "bad argument (null pointer, negative size, stride/dilation < 1, negative padding)",
    2: "channel mismatch or empty output window",
    3: "output dims are not [N, K, P, Q]",
    4: "a sum does not fit in int32",
}

_I64x4 = ctypes.c_int64 * 4
_I64x2 = ctypes.c_int64 * 2


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}: {_ERRORS.get(code, 'unknown')}")
        self.code = code


def _v4(v) -> ctypes.Array:
    v = [int(a) for a in v]
    assert len(v) == 4
    return _I64x4(*v)


def _v2(v) -> ctypes.Array:
    if isinstance(v, int):
        v = (v, v)
    v = [int(a) for a in v]
    assert len(v) == 2
    return _I64x2(*v)


class Oracle:
    """One loaded copy of the oracle library (tests may load mutated builds)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_out_dims.argtypes = [P] * 7
        lib.oracle_out_dims.restype = ctypes.c_int
        lib.oracle_conv_fprop.argtypes = [P] * 13 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_fprop.restype = ctypes.c_int
        lib.oracle_conv_fprop_points.argtypes = [P] * 10 + [ctypes.c_int, P, ctypes.c_int64, P]
        lib.oracle_conv_fprop_points.restype = ctypes.c_int
        lib.oracle_conv_fprop_requant.argtypes = [P] * 13 + [P, ctypes.c_float, P, ctypes.c_int,
                                                             ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_fprop_requant.restype = ctypes.c_int
        lib.oracle_requant_values.argtypes = [P, P, ctypes.c_int64, P, ctypes.c_float, P,
                                              ctypes.c_int, P]
        lib.oracle_requant_values.restype = ctypes.c_int
        lib.oracle_conv_dgrad.argtypes = [P] * 13 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_dgrad.restype = ctypes.c_int
        lib.oracle_conv_wgrad.argtypes = [P] * 13 + [ctypes.c_int, ctypes.c_int]
        lib.oracle_conv_wgrad.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def out_dims(self, xdims, wdims, pre, post, stride, dil):
        out = _I64x4()
        rc = self.lib.oracle_out_dims(_v4(xdims), _v4(wdims), _v2(pre), _v2(post),
                                      _v2(stride), _v2(dil), out)
        if rc:
            raise OracleError(rc)
        return tuple(int(a) for a in out)

    def conv_fprop(self, x: torch.Tensor, w: torch.Tensor, pre=0, post=0, stride=1, dil=1,
                   out: Optional[torch.Tensor] = None, threads: int = 0,
                   allow_overflow: bool = False, mode: int = 0) -> torch.Tensor:
        """Y = conv(x, w) as int32.  x, w: int8 CPU tensors with any strides.
        ``mode`` 0 is cross-correlation, 1 true convolution (flipped taps).

        ``out`` (int32, CPU, any non-overlapping strides) receives the result
        if given; otherwise a contiguous N,K,P,Q tensor is returned.
        """
        _check_cpu(x, torch.int8, "x")
        _check_cpu(w, torch.int8, "w")
        yd = self.out_dims(x.shape, w.shape, pre, post, stride, dil)
        if out is None:
            out = torch.empty(yd, dtype=torch.int32)
        _check_cpu(out, torch.int32, "out")
        if tuple(out.shape) != yd:
            raise OracleError(3)
        rc = self.lib.oracle_conv_fprop(
            ctypes.c_void_p(x.data_ptr()), _v4(x.shape), _v4(x.stride()),
            ctypes.c_void_p(w.data_ptr()), _v4(w.shape), _v4(w.stride()),
            ctypes.c_void_p(out.data_ptr()), _v4(out.shape), _v4(out.stride()),
            _v2(pre), _v2(post), _v2(stride), _v2(dil), int(mode), int(threads))
        if rc and not (rc == 4 and allow_overflow):
            raise OracleError(rc)
        return out

    def conv_fprop_points(self, x: torch.Tensor, w: torch.Tensor, idx, pre=0, post=0,
                          stride=1, dil=1, mode: int = 0) -> np.ndarray:
        """Exact int64 sums at the (n, k, p, q) rows of ``idx``."""
        _check_cpu(x, torch.int8, "x")
        _check_cpu(w, torch.int8, "w")
        idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
        res = np.empty(idx.shape[0], dtype=np.int64)
        rc = self.lib.oracle_conv_fprop_points(
            ctypes.c_void_p(x.data_ptr()), _v4(x.shape), _v4(x.stride()),
            ctypes.c_void_p(w.data_ptr()), _v4(w.shape), _v4(w.stride()),
            _v2(pre), _v2(post), _v2(stride), _v2(dil), int(mode),
            idx.ctypes.data_as(ctypes.c_void_p), ctypes.c_int64(idx.shape[0]),
            res.ctypes.data_as(ctypes.c_void_p))
        if rc:
            raise OracleError(rc)
        return res


    def conv_fprop_requant(self, x: torch.Tensor, w: torch.Tensor, pre=0, post=0, stride=1,
                           dil=1, scale=None, alpha: float = 1.0, bias=None, relu: bool = False,
                           out: Optional[torch.Tensor] = None, threads: int = 0,
                           mode: int = 0) -> torch.Tensor:
        """int8 Y = saturate(rint(relu?(fma(float(conv(x, w)), s_k, b_k)))).

        ``scale`` and ``bias`` are K floats (anything np.float32 accepts) or
        None (alpha for every channel, no bias).  ``out`` (int8, CPU, any
        non-overlapping strides) receives the result if given.
        """
        _check_cpu(x, torch.int8, "x")
        _check_cpu(w, torch.int8, "w")
        yd = self.out_dims(x.shape, w.shape, pre, post, stride, dil)
        if out is None:
            out = torch.empty(yd, dtype=torch.int8)
        _check_cpu(out, torch.int8, "out")
        if tuple(out.shape) != yd:
            raise OracleError(3)
        sc = _channel_floats(scale, yd[1], "scale")
        bi = _channel_floats(bias, yd[1], "bias")
        rc = self.lib.oracle_conv_fprop_requant(
            ctypes.c_void_p(x.data_ptr()), _v4(x.shape), _v4(x.stride()),
            ctypes.c_void_p(w.data_ptr()), _v4(w.shape), _v4(w.stride()),
            ctypes.c_void_p(out.data_ptr()), _v4(out.shape), _v4(out.stride()),
            _v2(pre), _v2(post), _v2(stride), _v2(dil),
            _ptr(sc), ctypes.c_float(alpha), _ptr(bi), int(bool(relu)), int(mode), int(threads))
        if rc:
            raise OracleError(rc)
        return out

    def requant_values(self, acc, ch, scale=None, alpha: float = 1.0, bias=None,
                       relu: bool = False) -> np.ndarray:
        """The requantising epilogue alone: int8 of each exact sum ``acc[i]``
        taken as output channel ``ch[i]``."""
        acc = np.ascontiguousarray(np.asarray(acc, dtype=np.int64).reshape(-1))
        ch = np.ascontiguousarray(np.broadcast_to(np.asarray(ch, dtype=np.int64), acc.shape))
        if acc.size and (ch.min() < 0 or ((scale is not None or bias is not None) and
                                          ch.max() >= _nchan(scale, bias))):
            raise OracleError(1)
        sc = None if scale is None else np.ascontiguousarray(np.asarray(scale, dtype=np.float32))
        bi = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
        res = np.empty(acc.shape, dtype=np.int8)
        rc = self.lib.oracle_requant_values(
            acc.ctypes.data_as(ctypes.c_void_p), ch.ctypes.data_as(ctypes.c_void_p),
            ctypes.c_int64(acc.size), _ptr(sc), ctypes.c_float(alpha), _ptr(bi),
            int(bool(relu)), res.ctypes.data_as(ctypes.c_void_p))
        if rc:
            raise OracleError(rc)
        return res


    def conv_dgrad(self, dy: torch.Tensor, w: torch.Tensor, dx_dims=None, pre=0, post=0,
                   stride=1, dil=1, out: Optional[torch.Tensor] = None, threads: int = 0,
                   mode: int = 0) -> torch.Tensor:
        """dX (int32 [N,C,H,W]) of the loss dY (int8 [N,K,P,Q]) through
        filter w (int8 [K,C,R,S]).  The image size comes from ``out`` or
        ``dx_dims`` (several H give the same P when the stride exceeds 1)."""
        _check_cpu(dy, torch.int8, "dy")
        _check_cpu(w, torch.int8, "w")
        if out is None:
            if dx_dims is None:
                raise ValueError("give dx_dims or out")
            out = torch.empty(tuple(dx_dims), dtype=torch.int32)
        _check_cpu(out, torch.int32, "out")
        rc = self.lib.oracle_conv_dgrad(
            ctypes.c_void_p(dy.data_ptr()), _v4(dy.shape), _v4(dy.stride()),
            ctypes.c_void_p(w.data_ptr()), _v4(w.shape), _v4(w.stride()),
            ctypes.c_void_p(out.data_ptr()), _v4(out.shape), _v4(out.stride()),
            _v2(pre), _v2(post), _v2(stride), _v2(dil), int(mode), int(threads))
        if rc:
            raise OracleError(rc)
        return out


    def conv_wgrad(self, x: torch.Tensor, dy: torch.Tensor, dw_dims=None, pre=0, post=0,
                   stride=1, dil=1, out: Optional[torch.Tensor] = None, threads: int = 0,
                   mode: int = 0) -> torch.Tensor:
        """dW (int32 [K,C,R,S]; R, S from ``out`` or ``dw_dims``) of the loss
        dY (int8 [N,K,P,Q]) for the image x (int8 [N,C,H,W])."""
        _check_cpu(x, torch.int8, "x")
        _check_cpu(dy, torch.int8, "dy")
        if out is None:
            if dw_dims is None:
                raise ValueError("give dw_dims or out")
            out = torch.empty(tuple(dw_dims), dtype=torch.int32)
        _check_cpu(out, torch.int32, "out")
        rc = self.lib.oracle_conv_wgrad(
            ctypes.c_void_p(x.data_ptr()), _v4(x.shape), _v4(x.stride()),
            ctypes.c_void_p(dy.data_ptr()), _v4(dy.shape), _v4(dy.stride()),
            ctypes.c_void_p(out.data_ptr()), _v4(out.shape), _v4(out.stride()),
            _v2(pre), _v2(post), _v2(stride), _v2(dil), int(mode), int(threads))
        if rc:
            raise OracleError(rc)
        return out


def _nchan(scale, bias) -> int:
    n = [len(np.asarray(v).reshape(-1)) for v in (scale, bias) if v is not None]
    return min(n)


def _channel_floats(v, k: int, name: str) -> Optional[np.ndarray]:
    if v is None:
        return None
    if isinstance(v, torch.Tensor):
        v = v.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
    if a.size != k:
        raise ValueError(f"{name}: expected {k} values, got {a.size}")
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_cpu(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or t.dtype != dtype or t.dim() != 4:
        raise TypeError(f"{name}: expected a 4-D CPU tensor of {dtype}")


_DEFAULT: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    """Load the oracle library, compiling it first if it is not built."""
    global _DEFAULT
    if path is not None:
        return Oracle(path)
    if _DEFAULT is None:
        if (not os.path.exists(_build.LIB) or
                os.path.getmtime(_build.SRC) > os.path.getmtime(_build.LIB)):
            _build.compile_oracle()
        _DEFAULT = Oracle(_build.LIB)
    return _DEFAULT


def out_dims(*a, **k):
    return load().out_dims(*a, **k)


def conv_fprop(*a, **k):
    return load().conv_fprop(*a, **k)


def conv_fprop_points(*a, **k):
    return load().conv_fprop_points(*a, **k)


def conv_fprop_requant(*a, **k):
    return load().conv_fprop_requant(*a, **k)


def requant_values(*a, **k):
    return load().requant_values(*a, **k)


def conv_dgrad(*a, **k):
    return load().conv_dgrad(*a, **k)


def conv_wgrad(*a, **k):
    return load().conv_wgrad(*a, **k)


def max_threads() -> int:
    return load().max_threads()
