"""GPU parity of true convolution (CONV_I8_MODE_CONVOLUTION) through the
general C entry, against the oracle's mode 1 (pinned to scipy's convolve2d):
byte-exact over the whole output buffer including guard bands."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

from .test_gpu_parity import FOOTPRINT_TILES, TILES, _fill
from .test_gpu_requant import channel_params

pytestmark = pytest.mark.gpu

GUARD = 64


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


def _dev():
    return torch.device("cuda:0")


def run_mode_check(ci8, x_storage, xspec, w_storage, wspec, ospec, pre, post, stride, dil,
                   mode=1, requant=None, label=""):
    """requant: None for INT32 output, else (scale, bias, relu) numpy arrays."""
    x_cpu = torch.as_strided(x_storage, xspec.dims, xspec.strides, xspec.offset)
    w_cpu = torch.as_strided(w_storage, wspec.dims, wspec.strides, wspec.offset)
    xg = wl.to_device(x_storage, xspec, _dev())[1]
    wg = wl.to_device(w_storage, wspec, _dev())[1]
    q8 = requant is not None
    dt = torch.int8 if q8 else torch.int32
    sentinel = 77 if q8 else wl.SENTINEL
    size = ospec.storage_size + 2 * GUARD
    buf = torch.full((size,), sentinel, dtype=dt, device=_dev())
    og = torch.as_strided(buf, ospec.dims, ospec.strides, ospec.offset + GUARD)
    print(f"[gpu] mode {mode} {label} x={xspec.dims}/{xspec.strides} w={wspec.dims}/{wspec.strides} "
          f"y={ospec.dims}/{ospec.strides} pre={pre} post={post} stride={stride} dil={dil} "
          f"requant={q8} tile={os.environ.get('CONV_I8_TILE', '-')}", flush=True)
    if q8:
        sc, bi, relu = requant
        ci8.conv_fprop_i8_mode(xg, wg, mode, og, torch.from_numpy(sc).to(_dev()), None,
                               torch.from_numpy(bi).to(_dev()), relu, pre, post, stride, dil)
    else:
        ci8.conv_fprop_i8_mode(xg, wg, mode, og, pre_padding=pre, post_padding=post,
                               stride=stride, dilation=dil)
    torch.cuda.synchronize()
    got = buf.cpu()
    ref = torch.full((size,), sentinel, dtype=dt)
    rv = torch.as_strided(ref, ospec.dims, ospec.strides, ospec.offset + GUARD)
    if q8:
        oracle.conv_fprop_requant(x_cpu, w_cpu, pre, post, stride, dil, scale=requant[0],
                                  bias=requant[1], relu=requant[2], out=rv, mode=mode)
    else:
        oracle.conv_fprop(x_cpu, w_cpu, pre, post, stride, dil, out=rv, mode=mode)
    if not torch.equal(got, ref):
        diff = (got != ref).nonzero().reshape(-1)
        raise AssertionError(f"{label}: {diff.numel()} elements differ, first at {diff[:5].tolist()}")
    return got


@pytest.mark.parametrize("name", wl.CASE_ORDER)
def test_workload_convolution_mode(ci8, name):
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base + 2)
    run_mode_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out, c.pre, c.post,
                   c.stride, c.dilation, label=name)


@pytest.mark.parametrize("name", ["bottleneck_3x3_n32_c128_28", "dilated_asym_n16_c96_64x48"])
def test_workload_convolution_mode_requant(ci8, name):
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base)
    K, C, R, S = c.filter.dims
    sc, bi = channel_params(K, C * R * S, seed=5)
    run_mode_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out, c.pre, c.post,
                   c.stride, c.dilation, requant=(sc, bi, True), label=name)


def test_cross_correlation_through_the_general_entry(ci8):
    """Mode 0 of the general entry gives the plain entry's bytes."""
    c = wl.case("dilated_asym_n16_c96_64x48")
    d = wl.make_inputs(c, c.seed_base)
    a = run_mode_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out, c.pre,
                       c.post, c.stride, c.dilation, mode=0, label="mode 0")
    xg = wl.to_device(d["x_storage"], c.image, _dev())[1]
    wg = wl.to_device(d["w_storage"], c.filter, _dev())[1]
    buf = torch.full((c.out.storage_size + 2 * GUARD,), wl.SENTINEL, dtype=torch.int32, device=_dev())
    og = torch.as_strided(buf, c.out.dims, c.out.strides, c.out.offset + GUARD)
    ci8.conv_fprop_i8(xg, wg, og, c.pre, c.post, c.stride, c.dilation)
    torch.cuda.synchronize()
    assert torch.equal(buf.cpu(), a)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("R,S,C,out_layout", [(3, 3, 128, "nhwc"), (3, 3, 64, "nchw"),
                                              (2, 3, 48, "nhwc"), (3, 1, 80, "nchw")])
def test_tile_shapes_convolution_mode(ci8, monkeypatch, tile, R, S, C, out_layout):
    """Every tile with reversed tap order, ragged M and K, asymmetric padding
    and stride; non-square filters on the im2col kernel."""
    if tile in FOOTPRINT_TILES and (C % 64 or R != 3 or S != 3):
        pytest.skip("the footprint kernel takes 3x3 filters and whole 64-channel blocks")
    monkeypatch.setenv("CONV_I8_TILE", tile)
    N, H, W, K = 3, 17, 13, 200
    pre, post, st, dl = (2, 1), (0, 1), (2, 1), (1, 1)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, S), wl.channels_last_strides((K, C, R, S)))
    od = oracle.out_dims(xs.dims, ws.dims, pre, post, st, dl)
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1),
                                               ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    if f["tile"] != tile:
        pytest.skip(f"{tile} does not take this problem (plan {f['tile']})")
    g = torch.Generator().manual_seed(C + R)
    xv = torch.randint(-128, 128, xs.dims, dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, ws.dims, dtype=torch.int8, generator=g)
    run_mode_check(ci8, _fill(xs, xv, 9), xs, _fill(ws, wv, 10), ws, os_, pre, post, st, dl,
                   label=f"tile {tile} {R}x{S} C={C} {out_layout}")


@pytest.mark.parametrize("tile", ["t256x128", "t128x128", "64x64x64", "128x128x64", "w256x128x64"])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("out_layout", ["nhwc", "nchw"])
def test_kmajor_filter_modes_and_requant(ci8, monkeypatch, tile, mode, out_layout):
    """Filters stored R, S, C, K, read k-major by the 3x3 tail tiles and the
    im2col tiles: both tap orders, INT32 output and the requantising
    epilogues, a ragged second column tile (K = 144)."""
    monkeypatch.setenv("CONV_I8_TILE", tile)
    N, C, H, W, K = 3, 128, 9, 12, 144
    pre, post, st, dl = (1, 1), (1, 1), (1, 1), (1, 1)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, 3, 3), (1, K, 3 * C * K, C * K))
    od = oracle.out_dims(xs.dims, ws.dims, pre, post, st, dl)
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    assert (f["tile"], f["filter_read"]) == (tile, "kmajor"), f
    g = torch.Generator().manual_seed(60 + mode)
    xv = torch.randint(-128, 128, xs.dims, dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, ws.dims, dtype=torch.int8, generator=g)
    xst, wst = _fill(xs, xv, 11), _fill(ws, wv, 12)
    run_mode_check(ci8, xst, xs, wst, ws, os_, pre, post, st, dl, mode=mode,
                   label=f"k-major {tile} {out_layout}")
    sc, bi = channel_params(K, C * 9, seed=6)
    run_mode_check(ci8, xst, xs, wst, ws, os_, pre, post, st, dl, mode=mode, requant=(sc, bi, True),
                   label=f"k-major requant {tile} {out_layout}")
