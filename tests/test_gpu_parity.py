"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Every comparison is bit-exact over the whole output, and the output buffer is
pre-filled with a sentinel so that unwritten elements, and writes outside the
descriptor's footprint (gaps of strided outputs, guard bands), are caught.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 64  # sentinel elements before and after every output footprint


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


def _dev():
    return torch.device("cuda:0")


def _to_dev(storage: torch.Tensor, spec: wl.TensorSpec):
    return wl.to_device(storage, spec, _dev())[1]


def _out_with_guards(spec: wl.TensorSpec):
    size = spec.storage_size
    buf = torch.full((size + 2 * GUARD,), wl.SENTINEL, dtype=torch.int32, device=_dev())
    view = torch.as_strided(buf, spec.dims, spec.strides, spec.offset + GUARD)
    return buf, view


def _covered_mask(spec: wl.TensorSpec) -> torch.Tensor:
    size = spec.storage_size
    mask = torch.zeros(size + 2 * GUARD, dtype=torch.bool)
    if all(d > 0 for d in spec.dims):
        idx = torch.as_strided(torch.arange(size + 2 * GUARD), spec.dims, spec.strides, spec.offset + GUARD)
        mask[idx.reshape(-1)] = True
    return mask


def run_and_check(ci8, x_storage, xspec, w_storage, wspec, ospec, pre, post, stride, dil,
                  label="", entry="ws"):
    """Run the library on device copies and compare with the oracle on the CPU copies."""
    x_cpu = torch.as_strided(x_storage, xspec.dims, xspec.strides, xspec.offset)
    w_cpu = torch.as_strided(w_storage, wspec.dims, wspec.strides, wspec.offset)
    xg = _to_dev(x_storage, xspec)
    wg = _to_dev(w_storage, wspec)
    buf, og = _out_with_guards(ospec)
    print(f"[gpu] {label} x={xspec.dims}/{xspec.strides} w={wspec.dims}/{wspec.strides} "
          f"y={ospec.dims}/{ospec.strides} pre={pre} post={post} stride={stride} dil={dil} "
          f"entry={entry} tile={os.environ.get('CONV_I8_TILE', '-')}", flush=True)
    if entry == "ws":
        ci8.conv_fprop_i8(xg, wg, og, pre, post, stride, dil)
    else:
        ci8.conv_fprop_i8_plain(xg, wg, og, pre, post, stride, dil)
    torch.cuda.synchronize()
    got = buf.cpu()
    ref_buf = torch.full_like(got, wl.SENTINEL)
    ref_view = torch.as_strided(ref_buf, ospec.dims, ospec.strides, ospec.offset + GUARD)
    if all(d > 0 for d in ospec.dims):
        oracle.conv_fprop(x_cpu, w_cpu, pre, post, stride, dil, out=ref_view)
    if not torch.equal(got, ref_buf):
        mask = _covered_mask(ospec)
        diff = got != ref_buf
        raise AssertionError(
            f"{label}: {int((diff & mask).sum())} computed outputs differ, "
            f"{int((diff & ~mask).sum())} writes outside the footprint")
    return got


# ---------------------------------------------------------------------------
# The workloads at full size, three seeds each.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("j", [0, 1, 2])
@pytest.mark.parametrize("name", wl.CASE_ORDER)
def test_workload_parity(ci8, name, j):
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base + j)
    run_and_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out,
                  c.pre, c.post, c.stride, c.dilation, label=f"{name} seed {c.seed_base + j}")


@pytest.mark.parametrize("name", ["tiny_5x5_r3", "dilated_asym_n16_c96_64x48"])
def test_plain_entry_allocates_its_workspace(ci8, name):
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base)
    run_and_check(ci8, d["x_storage"], c.image, d["w_storage"], c.filter, c.out,
                  c.pre, c.post, c.stride, c.dilation, label=name, entry="plain")


def test_forum_strides_give_identical_bytes(ci8):
    c = wl.case("tiny_5x5_r3")
    d = wl.make_inputs(c, c.seed_base)
    a = run_and_check(ci8, d["x_storage"], wl.TensorSpec((1, 1, 5, 5), (25, 25, 5, 1)),
                      d["w_storage"], wl.TensorSpec((1, 1, 3, 3), (9, 9, 3, 1)), c.out,
                      c.pre, c.post, c.stride, c.dilation, label="forum answer strides")
    b = run_and_check(ci8, d["x_storage"], wl.TensorSpec((1, 1, 5, 5), (25, 1, 5, 1)),
                      d["w_storage"], wl.TensorSpec((1, 1, 3, 3), (9, 1, 3, 1)), c.out,
                      c.pre, c.post, c.stride, c.dilation, label="forum repro strides")
    assert torch.equal(a, b)


def test_repeat_runs_identical(ci8):
    c = wl.case("large_channel_n64_c512_14")
    d = wl.make_inputs(c, c.seed_base)
    xg = _to_dev(d["x_storage"], c.image)
    wg = _to_dev(d["w_storage"], c.filter)
    outs = []
    for _ in range(3):
        _, og = wl.alloc_output(c.out, _dev())
        ci8.conv_fprop_i8(xg, wg, og, c.pre, c.post, c.stride, c.dilation)
        outs.append(og)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


# ---------------------------------------------------------------------------
# Every tile shape, on ragged problems (M and K not multiples of any tile),
# blocked and flat inner order, channel- and pixel-innermost outputs.
# ---------------------------------------------------------------------------
TILES = ["64x64x64", "128x64x64", "64x128x64", "128x128x64", "128x128x128", "256x128x64",
         "128x256x64", "w256x128x64", "w128x128x64", "w256x128x128", "w128x192x128", "f256x128", "fw256x128",
         "f128x128", "fk256x128", "fk128x128", "r256x128", "t256x128", "t128x128", "direct"]
FOOTPRINT_TILES = [t for t in TILES if t[0] in "frt"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("C,out_layout", [(128, "nhwc"), (48, "nchw"), (256, "nchw"), (80, "nhwc")])
def test_tile_shapes(ci8, monkeypatch, tile, C, out_layout):
    if tile in FOOTPRINT_TILES and C % 64:
        pytest.skip("the footprint kernel takes whole 64-channel blocks")
    monkeypatch.setenv("CONV_I8_TILE", tile)
    g = torch.Generator().manual_seed(C)
    N, H, W, K = 3, 17, 13, 200
    x = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    w = torch.randint(-128, 128, (K, C, 3, 3), dtype=torch.int8, generator=g)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)))
    od = (N, K, 9, 13)
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    xst = torch.empty(xs.storage_size, dtype=torch.int8)
    torch.as_strided(xst, xs.dims, xs.strides).copy_(x)
    wst = torch.empty(ws.storage_size, dtype=torch.int8)
    torch.as_strided(wst, ws.dims, ws.strides).copy_(w)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), (2, 1), (0, 1), (2, 1), (1, 1)))
    if tile in FOOTPRINT_TILES and f["tile"] != tile:
        pytest.skip("footprint does not fit this tile shape")
    assert f["tile"] == tile
    run_and_check(ci8, xst, xs, wst, ws, os_, (2, 1), (0, 1), (2, 1), (1, 1), label=f"tile {tile} C={C}")


# ---------------------------------------------------------------------------
# Random shapes, parameters and layouts.
# ---------------------------------------------------------------------------
def _layout(rng, dims, kind):
    n, c, h, w = dims
    if kind == "nchw":
        return wl.TensorSpec(dims, wl.contiguous_strides(dims))
    if kind == "nhwc":
        return wl.TensorSpec(dims, wl.channels_last_strides(dims))
    if kind == "nhwc_padded":       # channel-innermost rows with spare room
        cp = c + 16 * int(rng.integers(0, 3))
        wpad = w + int(rng.integers(0, 3))
        st = (h * wpad * cp, 1, wpad * cp, cp)
        return wl.TensorSpec(dims, st, offset=16 * int(rng.integers(0, 3)))
    if kind == "wide_view":          # every other element along w
        full = (n, c, h, 2 * w)
        st = wl.contiguous_strides(full)
        return wl.TensorSpec(dims, (st[0], st[1], st[2], 2), storage=n * c * h * 2 * w)
    if kind == "bcast_n":            # one image repeated over the batch
        st = wl.channels_last_strides(dims)
        return wl.TensorSpec(dims, (0, st[1], st[2], st[3]))
    if kind == "hwcn":               # batch innermost
        return wl.TensorSpec(dims, (1, h * w * n, w * n, n))
    raise ValueError(kind)


def _out_layout(rng, dims, kind):
    n, k, p, q = dims
    if kind == "nchw":
        return wl.TensorSpec(dims, wl.contiguous_strides(dims))
    if kind == "nhwc":
        return wl.TensorSpec(dims, wl.channels_last_strides(dims))
    if kind == "gapped":             # output rows with unused gaps between them
        kp = k + 3
        return wl.TensorSpec(dims, (p * (q + 1) * kp, 1, (q + 1) * kp, kp), offset=5)
    raise ValueError(kind)


def _fill(spec, values, seed):
    st = torch.randint(-128, 128, (spec.storage_size,), dtype=torch.int8,
                       generator=torch.Generator().manual_seed(seed))
    torch.as_strided(st, spec.dims, spec.strides, spec.offset).copy_(values)
    return st


@pytest.mark.parametrize("tile", [None, "direct"])
def test_random_problems(ci8, monkeypatch, tile):
    """Random shapes, parameters and layouts; with "direct" forced, the
    problems small enough for the direct kernel run on it (the others on the
    tile the planner picks)."""
    if tile:
        monkeypatch.setenv("CONV_I8_TILE", tile)
    rng = np.random.default_rng(2024 if tile is None else 77)
    done = 0
    while done < 120:
        N = int(rng.integers(1, 5))
        C = int(rng.choice([1, 3, 8, 16, 24, 32, 48, 64, 96, 100, 128, 160]))
        K = int(rng.integers(1, 140))
        H, W = int(rng.integers(1, 24)), int(rng.integers(1, 24))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        st = tuple(int(v) for v in rng.integers(1, 4, 2))
        dl = tuple(int(v) for v in rng.integers(1, 4, 2))
        pre = tuple(int(v) for v in rng.integers(0, 4, 2))
        post = tuple(int(v) for v in rng.integers(0, 4, 2))
        try:
            od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        except oracle.OracleError:
            continue
        xk = str(rng.choice(["nchw", "nhwc", "nhwc_padded", "wide_view", "bcast_n", "hwcn"]))
        wk = str(rng.choice(["nchw", "nhwc", "nhwc_padded"]))
        ok = str(rng.choice(["nchw", "nhwc", "gapped"]))
        xs, ws, os_ = _layout(rng, (N, C, H, W), xk), _layout(rng, (K, C, R, S), wk), _out_layout(rng, od, ok)
        g = torch.Generator().manual_seed(done)
        xv = torch.randint(-128, 128, (1 if xk == "bcast_n" else N, C, H, W), dtype=torch.int8, generator=g)
        xv = xv.expand(N, C, H, W)
        wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g)
        if xk == "bcast_n":
            st_ = torch.randint(-128, 128, (xs.storage_size,), dtype=torch.int8, generator=g)
            torch.as_strided(st_, (1, C, H, W), xs.strides).copy_(xv[:1])
            xst = st_
        else:
            xst = _fill(xs, xv, done + 1)
        wst = _fill(ws, wv, done + 2)
        run_and_check(ci8, xst, xs, wst, ws, os_, pre, post, st, dl,
                      label=f"random #{done} image {xk} filter {wk} out {ok}")
        done += 1


# ---------------------------------------------------------------------------
# Degenerate and limit cases.
# ---------------------------------------------------------------------------
def _dense_case(ci8, N, C, H, W, K, R, S, pre, post, st, dl, xval=None, wval=None, label=""):
    od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, S), wl.channels_last_strides((K, C, R, S)))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od))
    g = torch.Generator().manual_seed(N * 7 + C)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g) if xval is None else \
        torch.full((N, C, H, W), xval, dtype=torch.int8)
    wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g) if wval is None else \
        torch.full((K, C, R, S), wval, dtype=torch.int8)
    return run_and_check(ci8, _fill(xs, xv, 1), xs, _fill(ws, wv, 2), ws, os_, pre, post, st, dl, label=label)


def test_zero_channels_give_zeros(ci8):
    got = _dense_case(ci8, 2, 0, 5, 5, 3, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1), label="C=0")
    assert (got[GUARD:-GUARD] == 0).all()


def test_image_without_pixels_gives_zeros(ci8):
    got = _dense_case(ci8, 2, 16, 0, 4, 8, 1, 1, (1, 0), (1, 0), (1, 1), (1, 1), label="H=0 padded")
    assert (got[GUARD:-GUARD] == 0).all()


def test_empty_batch_and_filters_write_nothing(ci8):
    for (N, K) in [(0, 4), (3, 0)]:
        got = _dense_case(ci8, N, 16, 5, 5, K, 3, 3, (0, 0), (0, 0), (1, 1), (1, 1), label=f"N={N} K={K}")
        assert (got == wl.SENTINEL).all()


def test_largest_exact_reduction(ci8):
    # C*R*S = 14563*9 = 131067, every product +16384: the largest sums the
    # library accepts, 2147401728, just below 2^31
    got = _dense_case(ci8, 1, 14563, 3, 3, 2, 3, 3, (0, 0), (0, 0), (1, 1), (1, 1),
                      xval=-128, wval=-128, label="max reduction")
    assert int(got[GUARD]) == 16384 * 131067


def test_window_is_whole_image(ci8):
    _dense_case(ci8, 2, 32, 7, 9, 5, 7, 9, (0, 0), (0, 0), (1, 1), (1, 1), label="window = image")


def test_large_dilation_and_stride(ci8):
    _dense_case(ci8, 2, 16, 30, 31, 33, 3, 2, (5, 0), (0, 7), (4, 3), (9, 11), label="dil 9/11")


def test_single_output_channel_and_pixel_tails(ci8):
    _dense_case(ci8, 1, 64, 1, 1, 1, 1, 1, (0, 0), (0, 0), (1, 1), (1, 1), label="1x1 everything")
    _dense_case(ci8, 5, 16, 3, 3, 129, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1), label="K=129")


@pytest.mark.parametrize("C,R,tile", [(32, 3, None), (64, 3, "f128x128"), (64, 1, "pw64x64")])
def test_batch_split_over_launches(ci8, monkeypatch, C, R, tile):
    """Images 2 GiB apart: one launch per image keeps every buffer offset
    below 2^31 (im2col, footprint and 1x1 kernels)."""
    if tile:
        monkeypatch.setenv("CONV_I8_TILE", tile)
    gap = 1 << 31
    N, H, W, K = 2, 9, 10, 40
    dims = (N, C, H, W)
    cl = wl.channels_last_strides(dims)
    xs = wl.TensorSpec(dims, (gap, cl[1], cl[2], cl[3]))
    ws = wl.TensorSpec((K, C, R, R), wl.channels_last_strides((K, C, R, R)))
    od = oracle.out_dims(dims, (K, C, R, R), (1, 1), (1, 1), (1, 1), (1, 1))
    os_ = wl.TensorSpec(od, wl.contiguous_strides(od) if R == 3 else wl.channels_last_strides(od))
    x_storage = torch.zeros(xs.storage_size, dtype=torch.int8)
    g = torch.Generator().manual_seed(5)
    torch.as_strided(x_storage, dims, xs.strides).copy_(torch.randint(-128, 128, dims, dtype=torch.int8, generator=g))
    w_storage = _fill(ws, torch.randint(-128, 128, (K, C, R, R), dtype=torch.int8, generator=g), 3)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                               ci8.desc(os_.dims, os_.strides, 2), 1, 1, 1, 1))
    assert f["batch_chunk"] == "1"
    if tile:
        assert f["tile"] == tile, f
    run_and_check(ci8, x_storage, xs, w_storage, ws, os_, (1, 1), (1, 1), (1, 1), (1, 1),
                  label=f"batch split {tile or 'im2col'}")


# ---------------------------------------------------------------------------
# The 3x3 footprint kernel: tiles that span several images, strides,
# dilations, asymmetric padding, an odd number of 64-channel blocks (the last
# block pair runs one all-zero block), ragged M and K, both output layouts.
# ---------------------------------------------------------------------------
FOOTPRINT_CASES = [
    # N, C, H, W, K, R, S, stride, dil, pre, post
    (5, 64, 14, 14, 70, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1)),
    (2, 128, 9, 11, 130, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1)),
    (2, 64, 6, 10, 64, 3, 3, (1, 2), (1, 1), (0, 2), (1, 0)),
    (2, 192, 6, 6, 33, 3, 3, (1, 1), (2, 2), (2, 2), (2, 2)),
    (2, 64, 10, 8, 64, 3, 3, (2, 1), (2, 1), (2, 0), (2, 1)),
    (2, 64, 9, 9, 40, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1)),
    (7, 256, 5, 5, 96, 3, 3, (1, 1), (1, 1), (0, 0), (0, 0)),
    (1, 320, 40, 3, 128, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1)),
]


@pytest.mark.parametrize("tile", FOOTPRINT_TILES)
@pytest.mark.parametrize("case_i", range(len(FOOTPRINT_CASES)))
@pytest.mark.parametrize("out_layout", ["nhwc", "nchw"])
def test_footprint_kernel(ci8, monkeypatch, tile, case_i, out_layout):
    N, C, H, W, K, R, S, st, dl, pre, post = FOOTPRINT_CASES[case_i]
    monkeypatch.setenv("CONV_I8_TILE", tile)
    od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, S), wl.channels_last_strides((K, C, R, S)))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                                  ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    # every case is sized so that its footprint fits every footprint tile
    assert plan["tile"] == tile, plan
    assert plan["kernel"] == "footprint"
    g = torch.Generator().manual_seed(case_i)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g)
    run_and_check(ci8, _fill(xs, xv, 1), xs, _fill(ws, wv, 2), ws, os_, pre, post, st, dl,
                  label=f"footprint {tile} case {case_i}")


# Filters stored R, S, C, K (output channels contiguous, as the data
# gradient's view of a KRSC filter is): the 3x3 tail tiles read them in place,
# 128 output channels per input-channel row, and transpose them in LDS.  The
# cases with K % 16 == 0 and C % 64 == 0, plus a ragged column tile (K = 80).
KMAJOR_CASES = [FOOTPRINT_CASES[i] for i in (2, 4, 6, 7)] + [
    (3, 128, 11, 13, 80, 3, 3, (1, 1), (1, 1), (1, 1), (1, 1)),
]


def _rsck_strides(K, C, R, S):
    return (1, K, S * C * K, C * K)


@pytest.mark.parametrize("tile", ["t256x128", "t128x128"])
@pytest.mark.parametrize("case_i", range(len(KMAJOR_CASES)))
@pytest.mark.parametrize("out_layout", ["nhwc", "nchw"])
def test_footprint_kernel_kmajor_filter(ci8, monkeypatch, tile, case_i, out_layout):
    N, C, H, W, K, R, S, st, dl, pre, post = KMAJOR_CASES[case_i]
    monkeypatch.setenv("CONV_I8_TILE", tile)
    od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, S), _rsck_strides(K, C, R, S))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                                  ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    assert (plan["tile"], plan["filter_read"], plan["workspace"]) == (tile, "kmajor", "0"), plan
    g = torch.Generator().manual_seed(50 + case_i)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g)
    run_and_check(ci8, _fill(xs, xv, 1), xs, _fill(ws, wv, 2), ws, os_, pre, post, st, dl,
                  label=f"k-major filter {tile} case {case_i}")


# The im2col tiles of 64-channel stages over 64, 128 or 256 columns read such
# filters in place too (blocked order), with any filter size, stride and
# dilation: ragged column tiles, both output layouts.
KMAJOR_IM2COL_TILES = ["64x64x64", "128x64x64", "64x128x64", "128x128x64", "256x128x64", "128x256x64",
                       "w256x128x64", "w128x128x64"]
KMAJOR_IM2COL_CASES = [
    # N, C, H, W, K, R, S, stride, dil, pre, post
    (2, 64, 9, 11, 80, 1, 1, (1, 1), (1, 1), (0, 0), (0, 0)),
    (3, 128, 10, 7, 144, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1)),
    (2, 64, 12, 13, 48, 3, 5, (2, 1), (2, 2), (2, 1), (1, 3)),
    (1, 192, 6, 6, 272, 2, 3, (1, 1), (1, 1), (0, 1), (1, 0)),
]


@pytest.mark.parametrize("tile", KMAJOR_IM2COL_TILES)
@pytest.mark.parametrize("case_i", range(len(KMAJOR_IM2COL_CASES)))
@pytest.mark.parametrize("out_layout", ["nhwc", "nchw"])
def test_im2col_kmajor_filter(ci8, monkeypatch, tile, case_i, out_layout):
    N, C, H, W, K, R, S, st, dl, pre, post = KMAJOR_IM2COL_CASES[case_i]
    monkeypatch.setenv("CONV_I8_TILE", tile)
    od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, R, S), _rsck_strides(K, C, R, S))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if out_layout == "nhwc" else wl.contiguous_strides(od))
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                                  ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
    assert (plan["tile"], plan["filter_read"], plan["order"]) == (tile, "kmajor", "blocked"), plan
    g = torch.Generator().manual_seed(70 + case_i)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g)
    run_and_check(ci8, _fill(xs, xv, 1), xs, _fill(ws, wv, 2), ws, os_, pre, post, st, dl,
                  label=f"k-major filter {tile} case {case_i}")


def test_random_kmajor_filter_problems(ci8, monkeypatch):
    """Random layers with R, S, C, K filters, on the planner's own choice or
    on a tile drawn from those that read such filters k-major (a forced tile
    that does not apply falls back to the plan): C a multiple of 64, K of 16,
    strides, dilation, padding, both output layouts; at least a third of them
    k-major, on several tiles."""
    rng = np.random.default_rng(61)
    choices = [None, "t256x128", "t128x128", "64x128x64", "128x64x64", "128x128x64", "256x128x64",
               "128x256x64", "w256x128x64", "w128x128x64"]
    done = kmaj = 0
    seen = set()
    while done < 24:
        tile = choices[int(rng.integers(0, len(choices)))]
        if tile is None:
            monkeypatch.delenv("CONV_I8_TILE", raising=False)
        else:
            monkeypatch.setenv("CONV_I8_TILE", tile)
        N, C, K = int(rng.integers(1, 4)), 64 * int(rng.integers(1, 4)), 16 * int(rng.integers(1, 17))
        H, W = (int(v) for v in rng.integers(3, 20, 2))
        R, S = (3, 3) if done % 3 == 0 else tuple(int(v) for v in rng.integers(1, 5, 2))
        pre = tuple(int(v) for v in rng.integers(0, 3, 2))
        post = tuple(int(v) for v in rng.integers(0, 3, 2))
        st = tuple(int(v) for v in rng.integers(1, 3, 2))
        dl = tuple(int(v) for v in rng.integers(1, 3, 2))
        try:
            od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        except oracle.OracleError:
            continue
        xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
        ws = wl.TensorSpec((K, C, R, S), _rsck_strides(K, C, R, S))
        os_ = wl.TensorSpec(od, wl.channels_last_strides(od) if done % 2 else wl.contiguous_strides(od))
        plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1),
                                                      ci8.desc(ws.dims, ws.strides, 1),
                                                      ci8.desc(os_.dims, os_.strides, 2), pre, post, st, dl))
        kmaj += plan["filter_read"] == "kmajor"
        seen.add(plan["tile"])
        g = torch.Generator().manual_seed(900 + done)
        xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
        wv = torch.randint(-128, 128, (K, C, R, S), dtype=torch.int8, generator=g)
        run_and_check(ci8, _fill(xs, xv, 1), xs, _fill(ws, wv, 2), ws, os_, pre, post, st, dl,
                      label=f"random R,S,C,K filter {done} ({plan['tile']}, {plan['filter_read']})")
        done += 1
    assert kmaj >= 8 and len(seen) >= 4, (kmaj, seen)


# ---------------------------------------------------------------------------
# The 1x1 streaming kernel: ragged pixel counts (not a multiple of 32 or of a
# wave's four tiles), ragged output channels and channels, stride and padding
# (pixels that read only zeros), several images.
# ---------------------------------------------------------------------------
POINTWISE_CASES = [
    # N, C, H, W, K, stride, pre, post
    (3, 64, 13, 11, 64, (1, 1), (0, 0), (0, 0)),
    (2, 256, 9, 7, 50, (1, 1), (0, 0), (0, 0)),
    (4, 48, 10, 10, 33, (2, 2), (1, 0), (0, 1)),
    (1, 112, 5, 37, 128, (1, 3), (2, 1), (1, 2)),
    (5, 16, 6, 6, 7, (1, 1), (1, 1), (1, 1)),
]


@pytest.mark.parametrize("case_i", range(len(POINTWISE_CASES)))
@pytest.mark.parametrize("layout", ["nhwc", "nchw"])
def test_pointwise_kernel(ci8, monkeypatch, case_i, layout):
    N, C, H, W, K, st, pre, post = POINTWISE_CASES[case_i]
    fn = next(f for f in (1, 2, 4) if 32 * f >= K)
    ks = next(k for k in (2, 4, 8) if 32 * k >= (C + 15) // 16 * 16)
    monkeypatch.setenv("CONV_I8_TILE", f"pw{32 * fn}x{32 * ks}")
    od = oracle.out_dims((N, C, H, W), (K, C, 1, 1), pre, post, st, (1, 1))
    xs = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)) if layout == "nhwc"
                       else wl.contiguous_strides((N, C, H, W)))
    ws = wl.TensorSpec((K, C, 1, 1), wl.contiguous_strides((K, C, 1, 1)))
    os_ = wl.TensorSpec(od, wl.channels_last_strides(od))
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(xs.dims, xs.strides, 1), ci8.desc(ws.dims, ws.strides, 1),
                                                  ci8.desc(os_.dims, os_.strides, 2), pre, post, st, (1, 1)))
    assert plan["kernel"] == "pointwise", plan
    g = torch.Generator().manual_seed(100 + case_i)
    xv = torch.randint(-128, 128, (N, C, H, W), dtype=torch.int8, generator=g)
    wv = torch.randint(-128, 128, (K, C, 1, 1), dtype=torch.int8, generator=g)
    run_and_check(ci8, _fill(xs, xv, 3), xs, _fill(ws, wv, 4), ws, os_, pre, post, st, (1, 1),
                  label=f"pointwise case {case_i} {layout}")


def test_side_stream_workspace(ci8):
    """A call on a side stream whose operands need repacking: the wrapper's
    workspace belongs to that stream, so work queued on the current stream
    right after the call cannot be handed the same block while the side
    stream still uses it.  Repeated calls with a busy current stream in
    between all give the oracle's bytes."""
    c = wl.case("dilated_asym_n16_c96_64x48")
    d = wl.make_inputs(c, c.seed_base + 3)
    xg = _to_dev(d["x_storage"], c.image)
    wg = _to_dev(d["w_storage"], c.filter)
    ref = oracle.conv_fprop(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    print(f"[gpu] side-stream calls on {c.name}", flush=True)
    for i in range(4):
        y = ci8.conv_fprop_i8(xg, wg, None, c.pre, c.post, c.stride, c.dilation, stream=side)
        y.record_stream(side)
        # allocations and writes on the current stream while the side stream runs
        junk = torch.full((8 << 20,), i + 1, dtype=torch.uint8, device=_dev())
        junk.add_(1)
        outs.append(y)
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.cpu(), ref)
