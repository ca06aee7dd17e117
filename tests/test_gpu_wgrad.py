"""GPU parity of the weight gradient (conv_wgrad_i8) against the oracle's
wgrad (pinned to float64 autograd and the adjoint identity): bit-exact over
the whole dW buffer, guard bands included."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

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


def _rand_storage(spec, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-128, 128, (spec.storage_size,), dtype=torch.int8, generator=g)


def run_wgrad_check(ci8, x_storage, xspec, dy_storage, dyspec, dwspec, pre, post, st, dl, mode=0,
                    label="", entry="ws"):
    x_cpu = torch.as_strided(x_storage, xspec.dims, xspec.strides, xspec.offset)
    dy_cpu = torch.as_strided(dy_storage, dyspec.dims, dyspec.strides, dyspec.offset)
    xg = wl.to_device(x_storage, xspec, _dev())[1]
    dyg = wl.to_device(dy_storage, dyspec, _dev())[1]
    size = dwspec.storage_size + 2 * GUARD
    buf = torch.full((size,), wl.SENTINEL, dtype=torch.int32, device=_dev())
    dwg = torch.as_strided(buf, dwspec.dims, dwspec.strides, dwspec.offset + GUARD)
    print(f"[gpu] wgrad {label} x={xspec.dims}/{xspec.strides} dy={dyspec.dims}/{dyspec.strides} "
          f"dw={dwspec.dims}/{dwspec.strides} pre={pre} post={post} stride={st} dil={dl} "
          f"mode={mode} entry={entry}", flush=True)
    if entry == "ws":
        ci8.conv_wgrad_i8(xg, dyg, dwg, pre, post, st, dl, mode=mode)
    else:
        ci8.conv_wgrad_i8_plain(xg, dyg, dwg, pre, post, st, dl, mode=mode)
    torch.cuda.synchronize()
    got = buf.cpu()
    ref = torch.full((size,), wl.SENTINEL, dtype=torch.int32)
    rv = torch.as_strided(ref, dwspec.dims, dwspec.strides, dwspec.offset + GUARD)
    oracle.conv_wgrad(x_cpu, dy_cpu, None, pre, post, st, dl, out=rv, mode=mode)
    if not torch.equal(got, ref):
        diff = (got != ref).nonzero().reshape(-1)
        raise AssertionError(f"{label}: {diff.numel()} elements differ, first at {diff[:5].tolist()}: "
                             f"got {got[diff[:5]].tolist()} want {ref[diff[:5]].tolist()}")


@pytest.mark.parametrize("name,mode", [(n, 0) for n in wl.CASE_ORDER] +
                         [("tiny_5x5_r3", 1), ("downsample_s2_n8_c64_56", 1),
                          ("dilated_asym_n16_c96_64x48", 1)])
def test_workload_wgrad(ci8, name, mode):
    """The weight gradient of every workload: the workload's image, a loss in
    the forward output's layout, dW in the filter's layout."""
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base + 4)
    dyspec = wl.TensorSpec(c.out.dims, c.out.strides)
    dwspec = wl.TensorSpec(c.filter.dims, c.filter.strides)
    run_wgrad_check(ci8, d["x_storage"], c.image, _rand_storage(dyspec, 7 + mode), dyspec, dwspec,
                    c.pre, c.post, c.stride, c.dilation, mode=mode, label=name)


def test_random_wgrad_problems(ci8):
    """Strides, dilations, padding beyond the taps' reach (all-padding taps),
    non-square filters, NCHW/NHWC/KCRS/KRSC layouts, both modes."""
    rng = np.random.default_rng(53)
    done = 0
    while done < 40:
        N, K, C = int(rng.integers(1, 5)), int(rng.integers(1, 70)), int(rng.integers(1, 70))
        H, W = (int(v) for v in rng.integers(1, 20, 2))
        R, S = (int(v) for v in rng.integers(1, 6, 2))
        pre = tuple(int(v) for v in rng.integers(0, 6, 2))
        post = tuple(int(v) for v in rng.integers(0, 5, 2))
        st = tuple(int(v) for v in rng.integers(1, 5, 2))
        dl = tuple(int(v) for v in rng.integers(1, 4, 2))
        try:
            od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        except oracle.OracleError:
            continue
        lay = lambda d: (wl.channels_last_strides(d) if rng.integers(0, 2) else wl.contiguous_strides(d))
        xspec = wl.TensorSpec((N, C, H, W), lay((N, C, H, W)))
        dyspec = wl.TensorSpec(od, lay(od))
        dwspec = wl.TensorSpec((K, C, R, S), lay((K, C, R, S)))
        run_wgrad_check(ci8, _rand_storage(xspec, 300 + done), xspec, _rand_storage(dyspec, 400 + done),
                        dyspec, dwspec, pre, post, st, dl, mode=done % 2, label=f"random {done}",
                        entry="plain" if done % 5 == 0 else "ws")
        done += 1


@pytest.mark.parametrize("tile,mode", [("w256x128x64", 0), ("128x128x64", 1), ("256x128x64", 0)])
def test_wgrad_kmajor_loss(ci8, monkeypatch, tile, mode):
    """The large-channel layer's weight gradient on tiles that read the
    transposed loss (channels-last, 64 images: [K, N, P, Q] with K
    contiguous) in place, k-major, with the reduction split over workgroups
    into partial copies; both modes."""
    c = wl.case("large_channel_n64_c512_14")
    monkeypatch.setenv("CONV_I8_TILE", tile)
    d = wl.make_inputs(c, c.seed_base + 9)
    dyspec = wl.TensorSpec(c.out.dims, c.out.strides)
    dwspec = wl.TensorSpec(c.filter.dims, c.filter.strides)
    f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(ci8.desc(c.image.dims, c.image.strides, ci8.DT_INT8),
                                               ci8.desc(dyspec.dims, dyspec.strides, ci8.DT_INT8),
                                               ci8.desc(dwspec.dims, dwspec.strides, ci8.DT_INT32),
                                               c.pre, c.post, c.stride, c.dilation, mode=mode))
    assert (f["tile"], f["filter_read"], f["split_sum"]) == (tile, "kmajor", "partial"), f
    run_wgrad_check(ci8, d["x_storage"], c.image, _rand_storage(dyspec, 17 + mode), dyspec, dwspec,
                    c.pre, c.post, c.stride, c.dilation, mode=mode, label=f"k-major loss {tile}")


@pytest.mark.parametrize("N", [3, 6, 20, 32])
def test_wgrad_small_batch_transposes(ci8, N):
    """Channels-last operands with a small batch: the transposed views have
    the batch as their channels (16 or 32 packed), so one repack tile covers
    4 or 2 image positions, including a ragged last tile.  Stride 2 along W
    leaves the last image column unread, so the image view is cropped and its
    rows and columns do not merge into one run."""
    C, K, H, W = 24, 40, 7, 10
    xspec = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    od = oracle.out_dims((N, C, H, W), (K, C, 3, 3), (0, 0), (0, 0), (1, 2), (1, 1))
    dyspec = wl.TensorSpec(od, wl.channels_last_strides(od))
    dwspec = wl.TensorSpec((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)))
    run_wgrad_check(ci8, _rand_storage(xspec, 700 + N), xspec, _rand_storage(dyspec, 800 + N), dyspec, dwspec,
                    (0, 0), (0, 0), (1, 2), (1, 1), mode=N % 2, label=f"small batch {N}", entry="ws")


@pytest.mark.parametrize("layout,split_sum", [("kcrs_dense", "partial"), ("krsc_gaps", "atomic")])
def test_wgrad_split_paths(ci8, monkeypatch, capfd, layout, split_sum):
    """A weight gradient whose long N*P*Q reduction is split over workgroups
    (the bottleneck workload: 36 tiles, 7 splits): a dense dW takes the
    partial copies plus reduction, a dW with gaps between its pixels (a view
    into a buffer twice as wide) takes the zero-fill plus atomics path."""
    c = wl.case("bottleneck_3x3_n32_c128_28")
    d = wl.make_inputs(c, c.seed_base + 6)
    dyspec = wl.TensorSpec(c.out.dims, c.out.strides)
    K, C, R, S = c.filter.dims
    if layout == "kcrs_dense":
        dwspec = wl.TensorSpec((K, C, R, S), wl.contiguous_strides((K, C, R, S)))
    else:
        dwspec = wl.TensorSpec((K, C, R, S), (R * S * 2 * C, 1, S * 2 * C, 2 * C))
    monkeypatch.setenv("CONV_I8_LOG", "1")
    run_wgrad_check(ci8, d["x_storage"], c.image, _rand_storage(dyspec, 21), dyspec, dwspec,
                    c.pre, c.post, c.stride, c.dilation, label=f"split {layout}")
    logged = capfd.readouterr().err
    plans = [ci8.plan_fields(l) for l in logged.splitlines() if "ksplit=" in l]
    assert plans and all(p["split_sum"] == split_sum and int(p["ksplit"]) > 1 for p in plans), logged


# (N, C, K, H, W, x pitch or None (dense channels-last), dW layout, mode, ksplit > 1 expected)
WGRAD_1X1_CASES = [
    (2, 48, 80, 9, 11, None, "kcrs", 0, False),
    (2, 48, 80, 9, 11, None, "krsc", 1, False),
    (1, 272, 144, 20, 20, None, "kcrs", 0, False),     # ragged tiles along both K and C
    (4, 64, 32, 32, 32, None, "krsc", 0, True),        # 4096 pixels over several splits
    (3, 48, 96, 17, 23, 64, "kcrs", 1, True),          # image pixels 64 bytes apart (a channel slice)
    (1, 16, 16, 1, 1, None, "kcrs", 0, False),         # one pixel
]


@pytest.mark.parametrize("case", WGRAD_1X1_CASES)
def test_wgrad_1x1_in_place(ci8, case):
    """A 1x1 weight gradient of stride 1 without padding on channels-last
    operands: both read in place by the dedicated kernel (no repack), ragged
    tiles, one or several splits, a pixel pitch wider than the channels, both
    dW layouts and both modes."""
    N, C, K, H, W, pitch, dwl, mode, split = case
    xdims = (N, C, H, W)
    if pitch is None:
        xspec = wl.TensorSpec(xdims, wl.channels_last_strides(xdims))
    else:
        xspec = wl.TensorSpec(xdims, (H * W * pitch, 1, W * pitch, pitch))
    dydims = (N, K, H, W)
    dyspec = wl.TensorSpec(dydims, wl.channels_last_strides(dydims))
    dwdims = (K, C, 1, 1)
    dwspec = wl.TensorSpec(dwdims, wl.contiguous_strides(dwdims) if dwl == "kcrs" else wl.channels_last_strides(dwdims))
    zero, one = (0, 0), (1, 1)
    f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(ci8.desc(xdims, xspec.strides, ci8.DT_INT8),
                                               ci8.desc(dydims, dyspec.strides, ci8.DT_INT8),
                                               ci8.desc(dwdims, dwspec.strides, ci8.DT_INT32),
                                               zero, zero, one, one, mode=mode))
    assert f["kernel"] == "wgrad_in_place" and (int(f["ksplit"]) > 1) == split, f
    seed = N * 1000 + C + K
    run_wgrad_check(ci8, _rand_storage(xspec, seed), xspec, _rand_storage(dyspec, seed + 1), dyspec, dwspec,
                    zero, zero, one, one, mode=mode, label=f"1x1 in place {case}")
    run_wgrad_check(ci8, _rand_storage(xspec, seed + 2), xspec, _rand_storage(dyspec, seed + 3), dyspec, dwspec,
                    zero, zero, one, one, mode=mode, label=f"1x1 in place {case}, plain entry", entry="plain")


def test_random_wgrad_in_place_taps(ci8):
    """Random channels-last weight gradients (C and K multiples of 16) that
    the in-place kernel serves tap by tap: strides, dilations, padding on
    either side (taps that read only padding included), non-square filters,
    both dW layouts, both modes, one or several splits."""
    rng = np.random.default_rng(97)
    done = 0
    while done < 24:
        N = int(rng.integers(1, 5))
        C, K = 16 * int(rng.integers(1, 12)), 16 * int(rng.integers(1, 12))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        st = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dl = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        pre = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        post = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        if min(od) < 1:
            continue
        xspec = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
        dyspec = wl.TensorSpec(od, wl.channels_last_strides(od))
        dwd = (K, C, R, S)
        dwspec = wl.TensorSpec(dwd, wl.contiguous_strides(dwd) if done % 2 else wl.channels_last_strides(dwd))
        mode = int(rng.integers(0, 2))
        f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(ci8.desc(xspec.dims, xspec.strides, ci8.DT_INT8),
                                                   ci8.desc(od, dyspec.strides, ci8.DT_INT8),
                                                   ci8.desc(dwd, dwspec.strides, ci8.DT_INT32),
                                                   pre, post, st, dl, mode=mode))
        assert f["kernel"] == "wgrad_in_place", f
        run_wgrad_check(ci8, _rand_storage(xspec, 900 + done), xspec, _rand_storage(dyspec, 950 + done), dyspec,
                        dwspec, pre, post, st, dl, mode=mode, label=f"in place taps #{done} {f['image_rows']} "
                        f"ksplit {f['ksplit']}")
        done += 1
