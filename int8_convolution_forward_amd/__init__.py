"""INT8 conv_fprop for MI355X (gfx950): thin ctypes binding of libconv_i8.so.

Argument marshalling only: torch tensors are turned into the C descriptors
(logical dims + element strides, dtype), device pointers and the current HIP
stream, and every step of the convolution runs in the library's HIP kernels.
PyTorch provides the device memory (outputs, workspace) and the stream.

The operation is the one of the cuDNN "Convolutions" page ("Convolution
Fprop"): image [N,C,H,W] int8, weight [K,C,R,S] int8 -> [N,K,P,Q] int32, with
pre/post padding, stride and dilation as in its Python API list; the
symmetric ``padding`` overload sets pre = post.  The requantising entries
write int8 instead: fma(float(sum), scale[k], bias[k]), optional ReLU, round
half to even, saturate (see ``conv_fprop_i8_requant``).  If the compiled
library is missing this module raises on import: there is no fallback
implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Tuple, Union

import torch

from . import build as _build

__all__ = [
    "ConvI8Error", "conv_fprop_i8", "conv_fprop_i8_ws", "conv_fprop_i8_plain", "conv_fprop_i8_noalloc",
    "conv_fprop_i8_out_dims", "conv_fprop_i8_workspace_size", "conv_fprop_i8_plan",
    "conv_fprop_i8_requant", "conv_fprop_i8_requant_ws", "conv_fprop_i8_requant_plain",
    "conv_fprop_i8_requant_workspace_size", "Requant", "conv_fprop_i8_ex_ws",
    "conv_fprop_i8_ex_workspace_size", "conv_fprop_i8_mode", "conv_dgrad_i8",
    "conv_dgrad_i8_ws", "conv_dgrad_i8_workspace_size", "conv_dgrad_i8_plain", "conv_wgrad_i8",
    "conv_wgrad_i8_ws", "conv_wgrad_i8_workspace_size", "conv_wgrad_i8_plain", "conv_wgrad_i8_plan", "MODE_CROSS_CORRELATION",
    "MODE_CONVOLUTION",
    "status_string", "LIB_PATH", "DT_INT8", "DT_INT32", "MAX_REDUCTION", "lib",
]

# CONV_I8_LIB names another build of the library (the host-sanitizer test
# loads a host-only build with AddressSanitizer through it)
LIB_PATH = os.environ.get("CONV_I8_LIB") or _build.LIB
DT_INT8 = 1
DT_INT32 = 2
MAX_REDUCTION = 131071
MODE_CROSS_CORRELATION = 0
MODE_CONVOLUTION = 1

STATUS = {
    0: "CONV_I8_OK", 1: "CONV_I8_ERR_NULL", 2: "CONV_I8_ERR_DTYPE", 3: "CONV_I8_ERR_RANK",
    4: "CONV_I8_ERR_DIMS", 5: "CONV_I8_ERR_PARAM", 6: "CONV_I8_ERR_CHANNELS",
    7: "CONV_I8_ERR_OUT_DIMS", 8: "CONV_I8_ERR_STRIDES", 9: "CONV_I8_ERR_RANGE",
    10: "CONV_I8_ERR_WORKSPACE", 11: "CONV_I8_ERR_UNSUPPORTED", 12: "CONV_I8_ERR_HIP",
    13: "CONV_I8_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 16 << 20


class Desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("dims", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class Requant(ctypes.Structure):
    """conv_i8_requant_t: per-channel scale (or alpha), bias, ReLU flag."""
    _fields_ = [("scale", ctypes.c_void_p), ("alpha", ctypes.c_float),
                ("bias", ctypes.c_void_p), ("relu", ctypes.c_int32)]


class ConvI8Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code
        self.name = STATUS.get(code, str(code))


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run int8_convolution_forward_amd/build.py "
        "(or __graft_entry__.build()) first. There is no fallback implementation.")

lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_DP = ctypes.POINTER(Desc)
_V2 = ctypes.POINTER(ctypes.c_int64)

lib.conv_fprop_i8_out_dims.argtypes = [_DP, _DP, _V2, _V2, _V2, _V2, _V2]
lib.conv_fprop_i8_workspace_size.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                             ctypes.POINTER(ctypes.c_size_t)]
lib.conv_fprop_i8_ws.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, _P,
                                 ctypes.c_size_t, _P]
lib.conv_fprop_i8.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, _P]
lib.conv_fprop_i8_noalloc.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, _P]
lib.conv_fprop_i8_plan.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                   ctypes.c_char_p, ctypes.c_size_t]
lib.conv_i8_tile_names.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
lib.conv_i8_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint32, _P, _P]
_RQ = ctypes.POINTER(Requant)
lib.conv_fprop_i8_requant_workspace_size.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                                     ctypes.POINTER(ctypes.c_size_t)]
lib.conv_fprop_i8_requant_ws.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, _RQ, _P,
                                         ctypes.c_size_t, _P]
lib.conv_fprop_i8_requant.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, _RQ, _P]
lib.conv_fprop_i8_ex_workspace_size.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
lib.conv_fprop_i8_ex_ws.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, ctypes.c_int32,
                                    _RQ, _P, ctypes.c_size_t, _P]
lib.conv_dgrad_i8_workspace_size.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
lib.conv_dgrad_i8_ws.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, ctypes.c_int32, _P,
                                 ctypes.c_size_t, _P]
lib.conv_dgrad_i8.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, ctypes.c_int32, _P]
lib.conv_wgrad_i8_workspace_size.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2,
                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
lib.conv_wgrad_i8_ws.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, ctypes.c_int32, _P,
                                 ctypes.c_size_t, _P]
lib.conv_wgrad_i8.argtypes = [_DP, _P, _DP, _P, _DP, _P, _V2, _V2, _V2, _V2, ctypes.c_int32, _P]
lib.conv_wgrad_i8_plan.argtypes = [_DP, _P, _DP, _P, _DP, _V2, _V2, _V2, _V2, ctypes.c_int32,
                                   ctypes.c_char_p, ctypes.c_size_t]
lib.conv_i8_status_string.argtypes = [ctypes.c_int]
lib.conv_i8_status_string.restype = ctypes.c_char_p
for _f in ("conv_fprop_i8_out_dims", "conv_fprop_i8_workspace_size", "conv_fprop_i8_ws",
           "conv_fprop_i8", "conv_fprop_i8_noalloc", "conv_fprop_i8_plan", "conv_fprop_i8_requant_workspace_size",
           "conv_fprop_i8_requant_ws", "conv_fprop_i8_requant", "conv_fprop_i8_ex_workspace_size",
           "conv_fprop_i8_ex_ws", "conv_dgrad_i8_workspace_size", "conv_dgrad_i8_ws", "conv_dgrad_i8",
           "conv_wgrad_i8_workspace_size", "conv_wgrad_i8_ws", "conv_wgrad_i8", "conv_wgrad_i8_plan",
           "conv_i8_tile_names", "conv_i8_mfma_ceiling"):
    getattr(lib, _f).restype = ctypes.c_int


def status_string(code: int) -> str:
    return lib.conv_i8_status_string(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise ConvI8Error(code, status_string(code))


_DTYPES = {torch.int8: DT_INT8, torch.int32: DT_INT32}


def desc(t_or_dims, strides=None, dtype: Union[int, torch.dtype, None] = None, ndim: int = 4) -> Desc:
    """C descriptor from a tensor (its shape, element strides and dtype) or
    from explicit dims / strides / dtype code."""
    d = Desc()
    if isinstance(t_or_dims, torch.Tensor):
        t = t_or_dims
        dims, strides = tuple(t.shape), tuple(t.stride())
        dtype = _DTYPES.get(t.dtype, 0) if dtype is None else dtype
        ndim = t.dim()
    else:
        dims = tuple(t_or_dims)
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPES.get(dtype, 0)
    d.dtype = int(dtype or 0)
    d.ndim = int(ndim)
    for i in range(min(4, len(dims))):
        d.dims[i] = int(dims[i])
        d.strides[i] = int(strides[i])
    return d


def _pair(v) -> ctypes.Array:
    if isinstance(v, int):
        v = (v, v)
    v = tuple(int(a) for a in v)
    if len(v) != 2:
        raise ValueError("spatial parameters are [h, w] pairs")
    return (ctypes.c_int64 * 2)(*v)


def _params(pre_padding, post_padding, stride, dilation, padding):
    if padding is not None:
        pre_padding = post_padding = padding
    return _pair(pre_padding), _pair(post_padding), _pair(stride), _pair(dilation)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_one_gpu(**tensors) -> Optional[torch.device]:
    """Every tensor handed to a C entry that the kernels read or write must be
    GPU memory of one device: a host pointer dereferenced by a kernel faults
    the GPU.  Raises before any C call; returns the device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if not t.is_cuda:
            raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, but the other operands are on {dev}")
    return dev


def _workspace(n: int, device, stream) -> Optional[torch.Tensor]:
    """n bytes of workspace from torch's caching allocator, allocated on the
    stream the kernels run on, so the block is not handed to other work
    before that stream has run the call."""
    if not n:
        return None
    if stream is None:
        return torch.empty(n, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(n, dtype=torch.uint8, device=device)


def conv_fprop_i8_out_dims(x, w, pre_padding=0, post_padding=0, stride=1, dilation=1,
                           padding=None) -> Tuple[int, int, int, int]:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    out = (ctypes.c_int64 * 4)()
    _check(lib.conv_fprop_i8_out_dims(ctypes.byref(_as_desc(x)), ctypes.byref(_as_desc(w)),
                                      pre, post, st, dl, out))
    return tuple(int(v) for v in out)


def _as_desc(t) -> Desc:
    return t if isinstance(t, Desc) else desc(t)


def _out_like(x: torch.Tensor, dims, dtype=torch.int32) -> torch.Tensor:
    fmt = torch.contiguous_format
    if x.dim() == 4 and x.is_contiguous(memory_format=torch.channels_last) and not x.is_contiguous():
        fmt = torch.channels_last
    return torch.empty(dims, dtype=dtype, device=x.device, memory_format=fmt)


def conv_fprop_i8_workspace_size(x, w, out, pre_padding=0, post_padding=0, stride=1,
                                 dilation=1, padding=None) -> int:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    n = ctypes.c_size_t()
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    wp = _ptr(w) if isinstance(w, torch.Tensor) else None
    _check(lib.conv_fprop_i8_workspace_size(ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(w)),
                                            wp, ctypes.byref(_as_desc(out)), pre, post, st, dl,
                                            ctypes.byref(n)))
    return int(n.value)


def conv_fprop_i8_plan(x, w, out=None, pre_padding=0, post_padding=0, stride=1, dilation=1,
                       padding=None) -> str:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    if out is None:
        dims = conv_fprop_i8_out_dims(x, w, pre_padding, post_padding, stride, dilation, padding)
        out = desc(dims, _contig(dims), DT_INT32)
    buf = ctypes.create_string_buffer(512)
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    wp = _ptr(w) if isinstance(w, torch.Tensor) else None
    _check(lib.conv_fprop_i8_plan(ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(w)), wp,
                                  ctypes.byref(_as_desc(out)), pre, post, st, dl, buf, 512))
    return buf.value.decode()


def conv_i8_tile_names() -> list:
    buf = ctypes.create_string_buffer(4096)
    _check(lib.conv_i8_tile_names(buf, 4096))
    return buf.value.decode().split(",")


def conv_i8_mfma_ceiling(workgroups: int, iters: int, seed: int, out: torch.Tensor, stream=None) -> None:
    """One launch of the matrix-core calibration kernel (out: int32 GPU
    tensor of at least workgroups * 256 elements)."""
    _on_one_gpu(out=out)
    if out.dtype != torch.int32 or out.numel() < workgroups * 256:
        raise ValueError("out must hold workgroups * 256 int32 elements")
    _check(lib.conv_i8_mfma_ceiling(int(workgroups), int(iters), int(seed) & 0xffffffff, _ptr(out),
                                    _stream_handle(stream)))


def plan_fields(plan: str) -> dict:
    return dict(re.findall(r"(\w+)=(\S+)", plan))


def _contig(dims):
    s, acc = [], 1
    for d in reversed(dims):
        s.append(acc)
        acc *= d
    return tuple(reversed(s))


def _stream_handle(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def conv_fprop_i8_ws(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, workspace: Optional[torch.Tensor],
                     pre_padding=0, post_padding=0, stride=1, dilation=1, padding=None,
                     stream=None) -> torch.Tensor:
    """Direct call of the C entry with an explicit workspace tensor."""
    _on_one_gpu(x=x, w=w, out=out, workspace=workspace)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.conv_fprop_i8_ws(ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w),
                                ctypes.byref(desc(out)), _ptr(out), pre, post, st, dl,
                                ws_ptr, ctypes.c_size_t(ws_bytes), _stream_handle(stream)))
    return out


def conv_fprop_i8_plain(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, pre_padding=0,
                        post_padding=0, stride=1, dilation=1, padding=None, stream=None) -> torch.Tensor:
    """The C entry that takes its own workspace with hipMallocAsync."""
    _on_one_gpu(x=x, w=w, out=out)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    _check(lib.conv_fprop_i8(ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w),
                             ctypes.byref(desc(out)), _ptr(out), pre, post, st, dl,
                             _stream_handle(stream)))
    return out


def conv_fprop_i8_noalloc(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, pre_padding=0,
                          post_padding=0, stride=1, dilation=1, padding=None,
                          stream=None) -> torch.Tensor:
    """The C entry that allocates nothing: its workspace is the library's
    static per-GPU scratch array (calls overlapping on one GPU race on it)."""
    _on_one_gpu(x=x, w=w, out=out)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    _check(lib.conv_fprop_i8_noalloc(ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w),
                                     ctypes.byref(desc(out)), _ptr(out), pre, post, st, dl,
                                     _stream_handle(stream)))
    return out


def conv_fprop_i8(x: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
                  pre_padding=0, post_padding=0, stride=1, dilation=1, padding=None,
                  stream=None) -> torch.Tensor:
    """Y = conv_fprop(x, w) as int32 on x's device.

    x: int8 [N,C,H,W], w: int8 [K,C,R,S], any strides.  ``out`` (int32
    [N,K,P,Q], any non-overlapping strides) is written if given; otherwise a
    new tensor in x's memory format is returned.  The workspace, if needed, is
    a torch allocation on the stream the call runs on.
    """
    _on_one_gpu(x=x, w=w, out=out)
    if out is None:
        dims = conv_fprop_i8_out_dims(x, w, pre_padding, post_padding, stride, dilation, padding)
        out = _out_like(x, dims)
    n = conv_fprop_i8_workspace_size(x, w, out, pre_padding, post_padding, stride, dilation, padding)
    ws = _workspace(n, out.device, stream)
    return conv_fprop_i8_ws(x, w, out, ws, pre_padding, post_padding, stride, dilation, padding,
                            stream)


def _requant(scale, alpha, bias, relu) -> Requant:
    """The C parameter block; scale and bias are float32 device tensors of K
    values (the caller keeps them alive until the stream has run the call)."""
    for name, t in (("scale", scale), ("bias", bias)):
        if t is not None and (not isinstance(t, torch.Tensor) or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise TypeError(f"{name}: expected a contiguous float32 tensor")
    return Requant(_ptr(scale), float(alpha), _ptr(bias), 1 if relu else 0)


def _check_channels(w, t, name):
    if t is not None and t.numel() != w.shape[0]:
        raise ValueError(f"{name}: expected {w.shape[0]} values (one per output channel)")


def conv_fprop_i8_requant_workspace_size(x, w, out, pre_padding=0, post_padding=0, stride=1,
                                         dilation=1, padding=None) -> int:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    n = ctypes.c_size_t()
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    wp = _ptr(w) if isinstance(w, torch.Tensor) else None
    _check(lib.conv_fprop_i8_requant_workspace_size(
        ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(w)), wp, ctypes.byref(_as_desc(out)),
        pre, post, st, dl, ctypes.byref(n)))
    return int(n.value)


def conv_fprop_i8_requant_ws(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor,
                             workspace: Optional[torch.Tensor], scale=None, alpha: float = 1.0,
                             bias=None, relu: bool = False, pre_padding=0, post_padding=0,
                             stride=1, dilation=1, padding=None, stream=None) -> torch.Tensor:
    """Direct call of the requantising C entry with an explicit workspace."""
    _on_one_gpu(x=x, w=w, out=out, workspace=workspace, scale=scale, bias=bias)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    rq = _requant(scale, alpha, bias, relu)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.conv_fprop_i8_requant_ws(
        ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w), ctypes.byref(desc(out)),
        _ptr(out), pre, post, st, dl, ctypes.byref(rq), ws_ptr, ctypes.c_size_t(ws_bytes),
        _stream_handle(stream)))
    return out


def conv_fprop_i8_requant_plain(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor, scale=None,
                                alpha: float = 1.0, bias=None, relu: bool = False, pre_padding=0,
                                post_padding=0, stride=1, dilation=1, padding=None,
                                stream=None) -> torch.Tensor:
    """The requantising C entry that takes its own workspace (hipMallocAsync)."""
    _on_one_gpu(x=x, w=w, out=out, scale=scale, bias=bias)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    rq = _requant(scale, alpha, bias, relu)
    _check(lib.conv_fprop_i8_requant(
        ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w), ctypes.byref(desc(out)),
        _ptr(out), pre, post, st, dl, ctypes.byref(rq), _stream_handle(stream)))
    return out


def conv_fprop_i8_requant(x: torch.Tensor, w: torch.Tensor, scale: Optional[torch.Tensor] = None,
                          alpha: float = 1.0, bias: Optional[torch.Tensor] = None,
                          relu: bool = False, out: Optional[torch.Tensor] = None, pre_padding=0,
                          post_padding=0, stride=1, dilation=1, padding=None,
                          stream=None) -> torch.Tensor:
    """int8 Y = saturate(rint(relu?(fma(float(conv(x, w)), s_k, b_k)))).

    ``scale`` and ``bias``: float32 device tensors of K values, or None
    (``alpha`` for every channel; no bias).  ``out`` (int8 [N,K,P,Q], any
    non-overlapping strides) is written if given; otherwise a new tensor in
    x's memory format.  The fused epilogue of the from-scratch kernel page's
    roadmap (ReLU and quantisation after the convolution, INT8 store with the
    clamp of its naive loop).
    """
    _on_one_gpu(x=x, w=w, out=out, scale=scale, bias=bias)
    _check_channels(w, scale, "scale")
    _check_channels(w, bias, "bias")
    if out is None:
        dims = conv_fprop_i8_out_dims(x, w, pre_padding, post_padding, stride, dilation, padding)
        out = _out_like(x, dims, torch.int8)
    n = conv_fprop_i8_requant_workspace_size(x, w, out, pre_padding, post_padding, stride,
                                             dilation, padding)
    ws = _workspace(n, out.device, stream)
    return conv_fprop_i8_requant_ws(x, w, out, ws, scale, alpha, bias, relu, pre_padding,
                                    post_padding, stride, dilation, padding, stream)


def conv_fprop_i8_ex_workspace_size(x, w, out, pre_padding=0, post_padding=0, stride=1,
                                    dilation=1, padding=None, mode: int = 0) -> int:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    n = ctypes.c_size_t()
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    wp = _ptr(w) if isinstance(w, torch.Tensor) else None
    _check(lib.conv_fprop_i8_ex_workspace_size(
        ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(w)), wp, ctypes.byref(_as_desc(out)),
        pre, post, st, dl, int(mode), ctypes.byref(n)))
    return int(n.value)


def conv_fprop_i8_ex_ws(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor,
                        workspace: Optional[torch.Tensor], mode: int = 0,
                        requant: Optional[Requant] = None, pre_padding=0, post_padding=0, stride=1,
                        dilation=1, padding=None, stream=None) -> torch.Tensor:
    """The general C entry: ``mode`` (0 cross-correlation, 1 true convolution)
    and, for an int8 ``out``, the requantisation block from ``_requant`` (whose
    scale and bias arrays must be GPU memory of the same device)."""
    _on_one_gpu(x=x, w=w, out=out, workspace=workspace)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.conv_fprop_i8_ex_ws(
        ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(w)), _ptr(w), ctypes.byref(desc(out)),
        _ptr(out), pre, post, st, dl, int(mode),
        ctypes.byref(requant) if requant is not None else None, ws_ptr,
        ctypes.c_size_t(ws_bytes), _stream_handle(stream)))
    return out


def conv_fprop_i8_mode(x: torch.Tensor, w: torch.Tensor, mode: int, out: Optional[torch.Tensor] = None,
                       scale: Optional[torch.Tensor] = None, alpha: Optional[float] = None,
                       bias: Optional[torch.Tensor] = None, relu: bool = False, pre_padding=0,
                       post_padding=0, stride=1, dilation=1, padding=None,
                       stream=None) -> torch.Tensor:
    """conv_fprop in either mode.  INT32 output unless a requantisation is
    asked for (scale, alpha, bias or relu given), then INT8."""
    rq_on = scale is not None or alpha is not None or bias is not None or relu
    _on_one_gpu(x=x, w=w, out=out, scale=scale, bias=bias)
    _check_channels(w, scale, "scale")
    _check_channels(w, bias, "bias")
    if out is None:
        dims = conv_fprop_i8_out_dims(x, w, pre_padding, post_padding, stride, dilation, padding)
        out = _out_like(x, dims, torch.int8 if rq_on else torch.int32)
    rq = _requant(scale, 1.0 if alpha is None else alpha, bias, relu) if rq_on else None
    n = conv_fprop_i8_ex_workspace_size(x, w, out, pre_padding, post_padding, stride, dilation,
                                        padding, mode)
    ws = _workspace(n, out.device, stream)
    return conv_fprop_i8_ex_ws(x, w, out, ws, mode, rq, pre_padding, post_padding, stride,
                               dilation, padding, stream)


def conv_dgrad_i8_workspace_size(dy, w, dx, pre_padding=0, post_padding=0, stride=1, dilation=1,
                                 padding=None, mode: int = 0) -> int:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    n = ctypes.c_size_t()
    dp = _ptr(dy) if isinstance(dy, torch.Tensor) else None
    wp = _ptr(w) if isinstance(w, torch.Tensor) else None
    _check(lib.conv_dgrad_i8_workspace_size(
        ctypes.byref(_as_desc(dy)), dp, ctypes.byref(_as_desc(w)), wp, ctypes.byref(_as_desc(dx)),
        pre, post, st, dl, int(mode), ctypes.byref(n)))
    return int(n.value)


def conv_dgrad_i8_ws(dy: torch.Tensor, w: torch.Tensor, dx: torch.Tensor,
                     workspace: Optional[torch.Tensor], pre_padding=0, post_padding=0, stride=1,
                     dilation=1, padding=None, mode: int = 0, stream=None) -> torch.Tensor:
    """Direct call of the dgrad C entry with an explicit workspace."""
    _on_one_gpu(dy=dy, w=w, dx=dx, workspace=workspace)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.conv_dgrad_i8_ws(
        ctypes.byref(desc(dy)), _ptr(dy), ctypes.byref(desc(w)), _ptr(w), ctypes.byref(desc(dx)),
        _ptr(dx), pre, post, st, dl, int(mode), ws_ptr, ctypes.c_size_t(ws_bytes),
        _stream_handle(stream)))
    return dx


def conv_dgrad_i8_plain(dy: torch.Tensor, w: torch.Tensor, dx: torch.Tensor, pre_padding=0,
                        post_padding=0, stride=1, dilation=1, padding=None, mode: int = 0,
                        stream=None) -> torch.Tensor:
    """The dgrad C entry that takes its own workspace (hipMallocAsync)."""
    _on_one_gpu(dy=dy, w=w, dx=dx)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    _check(lib.conv_dgrad_i8(
        ctypes.byref(desc(dy)), _ptr(dy), ctypes.byref(desc(w)), _ptr(w), ctypes.byref(desc(dx)),
        _ptr(dx), pre, post, st, dl, int(mode), _stream_handle(stream)))
    return dx


def conv_dgrad_i8(dy: torch.Tensor, w: torch.Tensor, dx: torch.Tensor, pre_padding=0,
                  post_padding=0, stride=1, dilation=1, padding=None, mode: int = 0,
                  stream=None) -> torch.Tensor:
    """dX (int32 [N,C,H,W], written into ``dx``, which fixes H and W) of the
    loss dY (int8 [N,K,P,Q]) through the filter w (int8 [K,C,R,S])."""
    _on_one_gpu(dy=dy, w=w, dx=dx)
    n = conv_dgrad_i8_workspace_size(dy, w, dx, pre_padding, post_padding, stride, dilation,
                                     padding, mode)
    ws = _workspace(n, dx.device, stream)
    return conv_dgrad_i8_ws(dy, w, dx, ws, pre_padding, post_padding, stride, dilation, padding,
                            mode, stream)


def conv_wgrad_i8_workspace_size(x, dy, dw, pre_padding=0, post_padding=0, stride=1, dilation=1,
                                 padding=None, mode: int = 0) -> int:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    n = ctypes.c_size_t()
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    dp = _ptr(dy) if isinstance(dy, torch.Tensor) else None
    _check(lib.conv_wgrad_i8_workspace_size(
        ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(dy)), dp, ctypes.byref(_as_desc(dw)),
        pre, post, st, dl, int(mode), ctypes.byref(n)))
    return int(n.value)


def conv_wgrad_i8_plan(x, dy, dw, pre_padding=0, post_padding=0, stride=1, dilation=1,
                       padding=None, mode: int = 0) -> str:
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    buf = ctypes.create_string_buffer(512)
    xp = _ptr(x) if isinstance(x, torch.Tensor) else None
    dp = _ptr(dy) if isinstance(dy, torch.Tensor) else None
    _check(lib.conv_wgrad_i8_plan(
        ctypes.byref(_as_desc(x)), xp, ctypes.byref(_as_desc(dy)), dp, ctypes.byref(_as_desc(dw)),
        pre, post, st, dl, int(mode), buf, 512))
    return buf.value.decode()


def conv_wgrad_i8_ws(x: torch.Tensor, dy: torch.Tensor, dw: torch.Tensor,
                     workspace: Optional[torch.Tensor], pre_padding=0, post_padding=0, stride=1,
                     dilation=1, padding=None, mode: int = 0, stream=None) -> torch.Tensor:
    """Direct call of the wgrad C entry with an explicit workspace."""
    _on_one_gpu(x=x, dy=dy, dw=dw, workspace=workspace)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.conv_wgrad_i8_ws(
        ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(dy)), _ptr(dy), ctypes.byref(desc(dw)),
        _ptr(dw), pre, post, st, dl, int(mode), ws_ptr, ctypes.c_size_t(ws_bytes),
        _stream_handle(stream)))
    return dw


def conv_wgrad_i8_plain(x: torch.Tensor, dy: torch.Tensor, dw: torch.Tensor, pre_padding=0,
                        post_padding=0, stride=1, dilation=1, padding=None, mode: int = 0,
                        stream=None) -> torch.Tensor:
    """The wgrad C entry that takes its own workspace (hipMallocAsync)."""
    _on_one_gpu(x=x, dy=dy, dw=dw)
    pre, post, st, dl = _params(pre_padding, post_padding, stride, dilation, padding)
    _check(lib.conv_wgrad_i8(
        ctypes.byref(desc(x)), _ptr(x), ctypes.byref(desc(dy)), _ptr(dy), ctypes.byref(desc(dw)),
        _ptr(dw), pre, post, st, dl, int(mode), _stream_handle(stream)))
    return dw


def conv_wgrad_i8(x: torch.Tensor, dy: torch.Tensor, dw: torch.Tensor, pre_padding=0,
                  post_padding=0, stride=1, dilation=1, padding=None, mode: int = 0,
                  stream=None) -> torch.Tensor:
    """dW (int32 [K,C,R,S], written into ``dw``, which fixes R and S) from the
    image x (int8 [N,C,H,W]) and the loss dY (int8 [N,K,P,Q])."""
    _on_one_gpu(x=x, dy=dy, dw=dw)
    n = conv_wgrad_i8_workspace_size(x, dy, dw, pre_padding, post_padding, stride, dilation,
                                     padding, mode)
    ws = _workspace(n, dw.device, stream)
    return conv_wgrad_i8_ws(x, dy, dw, ws, pre_padding, post_padding, stride, dilation, padding,
                            mode, stream)
