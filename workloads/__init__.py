"""Seeded synthetic workloads for INT8 conv_fprop.

This module holds the workload table (dims, element strides and conv
parameters of each case) and the seeded generators that fill the image and
filter tensors.  It computes nothing of the convolution itself: output dims
are written down literally for each case, and both the oracle and the HIP
library are checked against them elsewhere.

Value recipe (shared by tests and the benchmark):
  * values are drawn with ``torch.randint(-128, 128, ...)`` (every int8 value,
    -128..127 inclusive) from a CPU ``torch.Generator`` seeded per tensor;
  * values are drawn in logical N,C,H,W order and only then placed into the
    case's memory layout, so every layout of one case holds the same values;
  * image seed = ``seed``, filter seed = ``seed + 500``, storage bytes that no
    logical element covers (the gaps of a strided view) are filled from
    ``seed + 900`` so that a kernel reading them gives a wrong answer;
  * the "worst-case magnitude" recipe sets the upper half of the batch of the
    image and the upper half of the output channels of the filter to -128.

The forum repro on the "INT8 convolution using cuDNN Python Frontend" page
draws its inputs with ``torch.randint(-128, 127)`` (upper bound exclusive);
here the full int8 range is used, as the case descriptions ask.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch

__all__ = [
    "TensorSpec", "ConvCase", "CASES", "CASE_ORDER", "case", "contiguous_strides",
    "channels_last_strides", "make_inputs", "alloc_output", "SENTINEL",
    "storage_elems",
]

# Output buffers are pre-filled with this value so that an untouched element
# can never pass for a computed zero (the forum page's output buffer started
# out as zeros, which hid which elements the library had written).
SENTINEL = 0x7EADBEEF


def contiguous_strides(dims: Sequence[int]) -> Tuple[int, ...]:
    s, acc = [], 1
    for d in reversed(dims):
        s.append(acc)
        acc *= d
    return tuple(reversed(s))


def channels_last_strides(dims: Sequence[int]) -> Tuple[int, ...]:
    n, c, h, w = dims
    return (h * w * c, 1, w * c, c)


def storage_elems(dims: Sequence[int], strides: Sequence[int], offset: int = 0) -> int:
    """Smallest buffer (in elements) that holds every addressed element."""
    if any(d == 0 for d in dims):
        return offset
    return offset + 1 + sum((d - 1) * s for d, s in zip(dims, strides))


@dataclass(frozen=True)
class TensorSpec:
    dims: Tuple[int, int, int, int]
    strides: Tuple[int, int, int, int]
    storage: Optional[int] = None   # buffer size in elements (default: tight)
    offset: int = 0                 # element offset of (0,0,0,0) in the buffer

    @property
    def storage_size(self) -> int:
        if self.storage is not None:
            return self.storage
        return storage_elems(self.dims, self.strides, self.offset)


@dataclass(frozen=True)
class ConvCase:
    name: str
    image: TensorSpec
    filter: TensorSpec
    out: TensorSpec
    pre: Tuple[int, int]
    post: Tuple[int, int]
    stride: Tuple[int, int]
    dilation: Tuple[int, int]
    recipe: str = "uniform"          # "uniform" | "half_min"
    seed_base: int = 0
    description: str = ""

    @property
    def ops(self) -> int:
        n, k, p, q = self.out.dims
        _, c, r, s = self.filter.dims
        return 2 * n * k * p * q * c * r * s


def _cl(dims):
    return TensorSpec(tuple(dims), channels_last_strides(dims))


def _nchw(dims):
    return TensorSpec(tuple(dims), contiguous_strides(dims))


CASES: Dict[str, ConvCase] = {}


def _add(c: ConvCase):
    CASES[c.name] = c


_add(ConvCase(
    name="tiny_5x5_r3",
    description="forum repro shape: 1x1x5x5 image, 1x1x3x3 filter, NCHW",
    image=TensorSpec((1, 1, 5, 5), (25, 25, 5, 1)),
    filter=TensorSpec((1, 1, 3, 3), (9, 9, 3, 1)),
    out=TensorSpec((1, 1, 3, 3), (9, 9, 3, 1)),
    pre=(0, 0), post=(0, 0), stride=(1, 1), dilation=(1, 1), seed_base=1000))
_add(ConvCase(
    name="downsample_s2_n8_c64_56",
    description="8x64x56x56 -> K=64, 3x3, stride 2, pad 1, NHWC",
    image=_cl((8, 64, 56, 56)), filter=_cl((64, 64, 3, 3)), out=_cl((8, 64, 28, 28)),
    pre=(1, 1), post=(1, 1), stride=(2, 2), dilation=(1, 1), seed_base=2000))
_add(ConvCase(
    name="pointwise_1x1_n32_c256_56",
    description="32x256x56x56 -> K=64, 1x1, stride 1, pad 0, NHWC",
    image=_cl((32, 256, 56, 56)), filter=_cl((64, 256, 1, 1)), out=_cl((32, 64, 56, 56)),
    pre=(0, 0), post=(0, 0), stride=(1, 1), dilation=(1, 1), seed_base=3000))
_add(ConvCase(
    name="bottleneck_3x3_n32_c128_28",
    description="32x128x28x28 -> K=128, 3x3, stride 1, pad 1, NHWC",
    image=_cl((32, 128, 28, 28)), filter=_cl((128, 128, 3, 3)), out=_cl((32, 128, 28, 28)),
    pre=(1, 1), post=(1, 1), stride=(1, 1), dilation=(1, 1), seed_base=3500))
_add(ConvCase(
    name="large_channel_n64_c512_14",
    description="64x512x14x14 -> K=512, 3x3, stride 1, pad 1, NHWC (MFMA-bound)",
    image=_cl((64, 512, 14, 14)), filter=_cl((512, 512, 3, 3)), out=_cl((64, 512, 14, 14)),
    pre=(1, 1), post=(1, 1), stride=(1, 1), dilation=(1, 1), seed_base=4000))
_add(ConvCase(
    name="dilated_asym_n16_c96_64x48",
    description=("16x96x64x48 strided NCHW view (W stride 2 into a 2x-wide buffer) -> "
                 "K=192, 3x5, stride [2,1], dilation [2,2], pre [2,1], post [1,3]; "
                 "half the batch / half the filters constant -128"),
    image=TensorSpec((16, 96, 64, 48), (589824, 6144, 96, 2), storage=16 * 96 * 64 * 96),
    filter=_nchw((192, 96, 3, 5)),
    out=_nchw((16, 192, 32, 44)),
    pre=(2, 1), post=(1, 3), stride=(2, 1), dilation=(2, 2), recipe="half_min",
    seed_base=5000))

CASE_ORDER: List[str] = list(CASES)


def case(name: str) -> ConvCase:
    return CASES[name]


def _randint8(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(-128, 128, tuple(shape), dtype=torch.int8, generator=g)


def _place(values_nchw: torch.Tensor, spec: TensorSpec, poison_seed: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Put logical NCHW ``values`` into a fresh buffer laid out as ``spec``.

    Returns (storage, view): storage is a 1-D int8 buffer of
    ``spec.storage_size`` elements whose uncovered bytes hold poison values;
    view is the strided 4-D view of it.
    """
    size = spec.storage_size
    storage = _randint8((size,), poison_seed) if size else torch.empty(0, dtype=torch.int8)
    view = torch.as_strided(storage, spec.dims, spec.strides, spec.offset)
    view.copy_(values_nchw)
    return storage, view


def logical_values(c: ConvCase, seed: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Image and filter values in logical N,C,H,W / K,C,R,S order."""
    x = _randint8(c.image.dims, seed)
    w = _randint8(c.filter.dims, seed + 500)
    if c.recipe == "half_min":
        x[x.shape[0] // 2:] = -128
        w[w.shape[0] // 2:] = -128
    elif c.recipe != "uniform":
        raise ValueError(f"unknown value recipe {c.recipe!r}")
    return x, w


def make_inputs(c: ConvCase, seed: int, image_spec: Optional[TensorSpec] = None,
                filter_spec: Optional[TensorSpec] = None):
    """Seeded CPU inputs for one case.

    Returns dict with ``x_storage``, ``x`` (strided view), ``w_storage``,
    ``w``.  ``image_spec`` / ``filter_spec`` override the case's layout while
    keeping the same logical values.
    """
    xv, wv = logical_values(c, seed)
    xs, x = _place(xv, image_spec or c.image, seed + 900)
    ws, w = _place(wv, filter_spec or c.filter, seed + 901)
    return {"x_storage": xs, "x": x, "w_storage": ws, "w": w}


def to_device(storage: torch.Tensor, spec: TensorSpec, device) -> Tuple[torch.Tensor, torch.Tensor]:
    """Copy a storage buffer to ``device`` and rebuild the strided view there."""
    d = storage.to(device)
    return d, torch.as_strided(d, spec.dims, spec.strides, spec.offset)


def alloc_output(spec: TensorSpec, device="cpu", fill: int = SENTINEL):
    """Sentinel-filled int32 output buffer laid out as ``spec``."""
    storage = torch.full((spec.storage_size,), fill, dtype=torch.int32, device=device)
    return storage, torch.as_strided(storage, spec.dims, spec.strides, spec.offset)
