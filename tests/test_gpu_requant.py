"""GPU parity of the requantising INT8 epilogue: the HIP library through the
C ABI against the CPU oracle (which is pinned to exact rational arithmetic),
byte for byte over the whole output buffer, guard bands included.

Each comparison runs twice with different sentinel bytes in the output
buffer, so an element the kernel fails to write cannot hide behind a result
that happens to equal the sentinel.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

from .test_gpu_parity import FOOTPRINT_TILES, POINTWISE_CASES, TILES, _fill, _out_layout

pytestmark = pytest.mark.gpu

GUARD = 64
SENTINELS = (90, -91)


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


def _dev():
    return torch.device("cuda:0")


def channel_params(K, crs, seed, signed=True):
    """Per-channel scales that put typical sums of random int8 operands
    around +-64 (so both rounding and saturation occur), and biases."""
    rng = np.random.default_rng(seed)
    typical = math.sqrt(max(crs, 1)) * 128 * 128 / 3
    sc = (rng.uniform(0.3, 1.7, K) * 64 / typical).astype(np.float32)
    if signed:
        sc *= rng.choice([-1, 1], K).astype(np.float32)
    bi = rng.uniform(-20, 20, K).astype(np.float32)
    return sc, bi


def run_requant_check(ci8, x_storage, xspec, w_storage, wspec, ospec, pre, post, stride, dil,
                      scale=None, alpha=1.0, bias=None, relu=False, label="", entry="ws"):
    x_cpu = torch.as_strided(x_storage, xspec.dims, xspec.strides, xspec.offset)
    w_cpu = torch.as_strided(w_storage, wspec.dims, wspec.strides, wspec.offset)
    xg = wl.to_device(x_storage, xspec, _dev())[1]
    wg = wl.to_device(w_storage, wspec, _dev())[1]
    sg = None if scale is None else torch.from_numpy(scale).to(_dev())
    bg = None if bias is None else torch.from_numpy(bias).to(_dev())
    size = ospec.storage_size + 2 * GUARD
    ref = None
    for sentinel in SENTINELS:
        buf = torch.full((size,), sentinel, dtype=torch.int8, device=_dev())
        og = torch.as_strided(buf, ospec.dims, ospec.strides, ospec.offset + GUARD)
        print(f"[gpu] requant {label} x={xspec.dims}/{xspec.strides} w={wspec.dims} "
              f"y={ospec.dims}/{ospec.strides} pre={pre} post={post} stride={stride} dil={dil} "
              f"scale={'array' if scale is not None else alpha} bias={bias is not None} "
              f"relu={relu} entry={entry} tile={os.environ.get('CONV_I8_TILE', '-')}", flush=True)
        if entry == "ws":
            ci8.conv_fprop_i8_requant(xg, wg, sg, alpha, bg, relu, og, pre, post, stride, dil)
        else:
            ci8.conv_fprop_i8_requant_plain(xg, wg, og, sg, alpha, bg, relu, pre, post, stride, dil)
        torch.cuda.synchronize()
        got = buf.cpu()
        if ref is None:
            ref = torch.empty(size, dtype=torch.int8)
        ref.fill_(sentinel)
        rv = torch.as_strided(ref, ospec.dims, ospec.strides, ospec.offset + GUARD)
        if all(d > 0 for d in ospec.dims):
            oracle.conv_fprop_requant(x_cpu, w_cpu, pre, post, stride, dil, scale=scale,
                                      alpha=alpha, bias=bias, relu=relu, out=rv)
        if not torch.equal(got, ref):
            diff = (got != ref).nonzero().reshape(-1)
            raise AssertionError(f"{label} (sentinel {sentinel}): {diff.numel()} bytes differ, "
                                 f"first at {diff[:5].tolist()}: got {got[diff[:5]].tolist()} "
                                 f"want {ref[diff[:5]].tolist()}")
    return got


# ---------------------------------------------------------------------------
# The workloads at full size, with their own layouts.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", wl.CASE_ORDER)
def test_workload_requant(ci8, name):
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base)
    K, C, R, S = c.filter.dims
    sc, bi = channel_params(K, C * R * S, seed=len(name))
    run_requant_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out, c.pre,
                      c.post, c.stride, c.dilation, scale=sc, bias=bi, relu=(len(name) % 2 == 0),
                      label=name)


@pytest.mark.parametrize("relu", [False, True])
def test_scalar_alpha_and_plain_entry(ci8, relu):
    """alpha for every channel, no bias; the entry that allocates its own
    workspace (the dilated workload needs repacks)."""
    c = wl.case("dilated_asym_n16_c96_64x48")
    d = wl.make_inputs(c, c.seed_base + 1)
    run_requant_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out, c.pre,
                      c.post, c.stride, c.dilation, alpha=-3.0e-4, relu=relu,
                      label="alpha", entry="plain")


def test_unit_scale_is_the_saturating_store(ci8):
    """alpha 1, no bias, no ReLU: the INT8 result is the INT32 result clamped
    to [-128, 127] (the naive loop's store), on the GPU's own INT32 output."""
    c = wl.case("bottleneck_3x3_n32_c128_28")
    d = wl.make_inputs(c, c.seed_base)
    xg = wl.to_device(d["x_storage"], c.image, _dev())[1]
    wg = wl.to_device(d["w_storage"], c.filter, _dev())[1]
    y32 = ci8.conv_fprop_i8(xg, wg, None, c.pre, c.post, c.stride, c.dilation)
    y8 = ci8.conv_fprop_i8_requant(xg, wg, None, 1.0, None, False, None, c.pre, c.post,
                                   c.stride, c.dilation)
    torch.cuda.synchronize()
    assert torch.equal(y8.cpu(), y32.cpu().clamp(-128, 127).to(torch.int8))


# ---------------------------------------------------------------------------
# Every tile shape on a ragged problem, channel- and pixel-innermost outputs.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("C,K,out_layout", [(128, 200, "nhwc"), (64, 200, "nchw"), (48, 200, "gapped"),
                                            (64, 202, "nhwc"), (128, 200, "nhwc_off1")])
def test_tile_shapes_requant(ci8, monkeypatch, tile, C, K, out_layout):
    """nhwc with K % 4 == 0 takes the dword-packed stores; K = 202 and an
    output that starts at an odd byte take the byte stores."""
    if tile in FOOTPRINT_TILES and C % 64:
        pytest.skip("the footprint kernel takes whole 64-channel blocks")
    monkeypatch.setenv("CONV_I8_TILE", tile)
    N, H, W = 3, 17, 13
    pre, post, st, dl = (2, 1), (0, 1), (2, 1), (1, 1)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)))
    od = oracle.out_dims(xs.dims, ws.dims, pre, post, st, dl)
    if out_layout == "nhwc_off1":
        os_ = wl.TensorSpec(od, wl.channels_last_strides(od), offset=1)
    else:
        os_ = _out_layout(np.random.default_rng(0), od, out_layout)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1),
                                               ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    if f["tile"] != tile:
        pytest.skip(f"{tile} does not take this problem (plan {f['tile']})")
    g = torch.Generator().manual_seed(C + 7)
    xv = torch.randint(-128, 128, xs.dims, dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, ws.dims, dtype=torch.int8, generator=g)
    sc, bi = channel_params(K, C * 9, seed=C)
    run_requant_check(ci8, _fill(xs, xv, 5), xs, _fill(ws, wv, 6), ws, os_, pre, post, st, dl,
                      scale=sc, bias=bi, relu=(C == 64),
                      label=f"tile {tile} C={C} K={K} {out_layout}")


@pytest.mark.parametrize("case_i", range(len(POINTWISE_CASES)))
def test_pointwise_requant(ci8, monkeypatch, case_i):
    N, C, H, W, K, st, pre, post = POINTWISE_CASES[case_i]
    fn = next(f for f in (1, 2, 4) if 32 * f >= K)
    ks = next(k for k in (2, 4, 8) if 32 * k >= (C + 15) // 16 * 16)
    monkeypatch.setenv("CONV_I8_TILE", f"pw{32 * fn}x{32 * ks}")
    od = oracle.out_dims((N, C, H, W), (K, C, 1, 1), pre, post, st, (1, 1))
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, 1, 1), wl.contiguous_strides((K, C, 1, 1)))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od))
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1),
                                                  ci8.desc(ws.dims, ws.strides, 1),
                                                  ci8.desc(os_.dims, os_.strides, 2), pre, post, st,
                                                  (1, 1)))
    assert plan["kernel"] == "pointwise", plan
    g = torch.Generator().manual_seed(200 + case_i)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, (K, C, 1, 1), dtype=torch.int8, generator=g)
    sc, bi = channel_params(K, C, seed=case_i)
    run_requant_check(ci8, _fill(xs, xv, 7), xs, _fill(ws, wv, 8), ws, os_, pre, post, st, (1, 1),
                      scale=sc, bias=bi, relu=bool(case_i % 2), label=f"pointwise case {case_i}")


@pytest.mark.parametrize("tile", [None, "f128x128", "pw64x128"])
@pytest.mark.parametrize("relu", [False, True])
def test_nonfinite_scale_and_bias(ci8, monkeypatch, tile, relu):
    """Infinite and NaN scales and biases: a NaN after the multiply-add is
    written as 0, infinities saturate (the oracle's reading, pinned on the
    CPU).  Channel 0's filter is all zeros, so inf * 0 = NaN occurs; the
    other channels see signed infinities, NaN scales and biases, and
    infinities of opposite sign."""
    if tile:
        monkeypatch.setenv("CONV_I8_TILE", tile)
    R = 1 if tile and tile.startswith("pw") else 3
    N, C, H, W, K = 2, 64, 9, 7, 16
    pad = (R - 1) // 2
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, R), wl.channels_last_strides((K, C, R, R)))
    od = oracle.out_dims(xs.dims, ws.dims, (pad, pad), (pad, pad), (1, 1), (1, 1))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od))
    g = torch.Generator().manual_seed(41)
    xv = torch.randint(-128, 128, xs.dims, dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, ws.dims, dtype=torch.int8, generator=g)
    wv[0] = 0
    inf, nan = np.float32("inf"), np.float32("nan")
    sc = np.array([inf, inf, -inf, nan, 0.01, 0.01, 0.01, inf, -inf, nan, 1e30, -1e30, 0.02, inf, 0.0, inf],
                  dtype=np.float32)
    bi = np.array([0, 0, 1, 0, nan, inf, -inf, -inf, -inf, 5, 0, 0, nan, nan, inf, inf], dtype=np.float32)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), (pad, pad), (pad, pad),
                                               (1, 1), (1, 1)))
    if tile:
        assert f["tile"] == tile, f
    run_requant_check(ci8, _fill(xs, xv, 7), xs, _fill(ws, wv, 8), ws, os_, (pad, pad), (pad, pad),
                      (1, 1), (1, 1), scale=sc, bias=bi, relu=relu, label=f"nonfinite {tile}")
