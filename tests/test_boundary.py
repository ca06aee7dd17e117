"""The C-ABI boundary on the CPU: the library loads, exports every declared
symbol, and refuses bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest
import torch

import int8_convolution_forward_amd as ci8
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_i8.h")

# A non-null, 256-byte aligned address that is never dereferenced: every call
# below fails validation before any HIP call is made.
FAKE = ctypes.c_void_p(0x1000000)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(conv_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"conv_fprop_i8", "conv_fprop_i8_ws", "conv_fprop_i8_out_dims",
            "conv_fprop_i8_workspace_size", "conv_fprop_i8_plan", "conv_i8_status_string"} <= set(names)
    lib = ctypes.CDLL(ci8.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in ci8.STATUS.items():
        assert ci8.status_string(code).startswith(name)
    assert "unknown" in ci8.status_string(99)


def _args(c: wl.ConvCase, **over):
    a = dict(x=ci8.desc(c.image.dims, c.image.strides, ci8.DT_INT8),
             w=ci8.desc(c.filter.dims, c.filter.strides, ci8.DT_INT8),
             y=ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT32),
             pre=c.pre, post=c.post, stride=c.stride, dil=c.dilation)
    a.update(over)
    return a


def _call_ws(a, ws_bytes=0, ws=None, xp=FAKE, wp=FAKE, yp=FAKE):
    p = ci8._params(a["pre"], a["post"], a["stride"], a["dil"], None)
    return ci8.lib.conv_fprop_i8_ws(
        ctypes.byref(a["x"]) if a["x"] is not None else None, xp,
        ctypes.byref(a["w"]) if a["w"] is not None else None, wp,
        ctypes.byref(a["y"]) if a["y"] is not None else None, yp,
        *p, ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("name", wl.CASE_ORDER)
def test_out_dims_match_case_table(name):
    c = wl.case(name)
    d = _args(c)
    assert ci8.conv_fprop_i8_out_dims(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation) == c.out.dims


def test_printed_shapes():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "printed_shapes.json")) as f:
        for g in json.load(f)["cases"]:
            x = ci8.desc(g["image"], wl.contiguous_strides(g["image"]), ci8.DT_INT8)
            w = ci8.desc(g["filter"], wl.contiguous_strides(g["filter"]), ci8.DT_INT8)
            assert list(ci8.conv_fprop_i8_out_dims(x, w, g["pre"], g["post"], g["stride"],
                                                    g["dilation"])) == g["out"]


def test_int8_output_is_refused():
    """The forum repro left Y at the graph's INT8 io type and got saturated
    int8 bytes in its int32 buffer; here an INT8 output descriptor is an error."""
    c = wl.case("tiny_5x5_r3")
    a = _args(c, y=ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT8))
    assert _call_ws(a) == 2  # CONV_I8_ERR_DTYPE


def test_forum_strides_are_equivalent():
    """With C = 1 the channel stride never multiplies a nonzero index: the
    repro's [25,1,5,1] and the answer's [25,25,5,1] describe the same tensor."""
    c = wl.case("tiny_5x5_r3")
    p1 = ci8.conv_fprop_i8_plan(ci8.desc((1, 1, 5, 5), (25, 1, 5, 1), 1), ci8.desc((1, 1, 3, 3), (9, 1, 3, 1), 1))
    p2 = ci8.conv_fprop_i8_plan(ci8.desc((1, 1, 5, 5), (25, 25, 5, 1), 1), ci8.desc((1, 1, 3, 3), (9, 9, 3, 1), 1))
    assert p1 == p2


@pytest.mark.parametrize("over,code", [
    (dict(x=None), 1),
    (dict(y=None), 1),
    (dict(pre=(-1, 0)), 5),
    (dict(post=(0, -2)), 5),
    (dict(stride=(0, 1)), 5),
    (dict(dil=(1, 0)), 5),
])
def test_param_errors(over, code):
    assert _call_ws(_args(wl.case("downsample_s2_n8_c64_56"), **over)) == code


def test_descriptor_errors():
    c = wl.case("downsample_s2_n8_c64_56")
    x, w, y = c.image, c.filter, c.out
    D = ci8.desc
    cases = [
        (dict(x=D(x.dims, x.strides, ci8.DT_INT8, ndim=3)), 3),
        (dict(x=D(x.dims, x.strides, ci8.DT_INT32)), 2),
        (dict(w=D(w.dims, w.strides, 0)), 2),
        (dict(y=D(y.dims, y.strides, ci8.DT_INT8)), 2),
        (dict(x=D((8, 64, -1, 56), x.strides, ci8.DT_INT8)), 4),
        (dict(w=D((64, 64, 0, 3), w.strides, ci8.DT_INT8)), 4),
        (dict(w=D((64, 32, 3, 3), w.strides, ci8.DT_INT8)), 6),
        (dict(y=D((8, 64, 28, 29), y.strides, ci8.DT_INT32)), 7),
        (dict(y=D((8, 32, 28, 28), y.strides, ci8.DT_INT32)), 7),
        (dict(x=D((8, 64, 1, 1), (64, 1, 64, 64), ci8.DT_INT8), y=D((8, 64, 2, 2), (256, 1, 128, 64), ci8.DT_INT32)), 7),
        (dict(x=D(x.dims, (200704, 1, 3584, -64), ci8.DT_INT8)), 8),
        (dict(y=D(y.dims, (50176, 1, 1792, 32), ci8.DT_INT32)), 8),   # q and k overlap
        (dict(y=D(y.dims, (0, 1, 1792, 64), ci8.DT_INT32)), 8),       # batch overlaps
    ]
    for over, code in cases:
        assert _call_ws(_args(c, **over)) == code, (over, code)


def test_reduction_range():
    D = ci8.desc
    ok_c, bad_c = 14563, 14564      # 14563*9 = 131067 <= 131071 < 14564*9
    for C, code in [(ok_c, 10), (bad_c, 9)]:
        a = dict(x=D((1, C, 3, 3), (9 * C, 9, 3, 1), 1), w=D((1, C, 3, 3), (9 * C, 9, 3, 1), 1),
                 y=D((1, 1, 1, 1), (1, 1, 1, 1), 2), pre=0, post=0, stride=1, dil=1)
        # the allowed size gets as far as the workspace check (NCHW needs a repack)
        assert _call_ws(a) == code


def test_workspace_errors():
    c = wl.case("dilated_asym_n16_c96_64x48")
    a = _args(c)
    need = ci8.conv_fprop_i8_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation)
    assert need >= 16 * 64 * 48 * 96 + 192 * 15 * 96
    assert _call_ws(a, ws_bytes=need - 1, ws=FAKE) == 10
    assert _call_ws(a, ws_bytes=need, ws=None) == 1
    assert _call_ws(a, ws_bytes=need, ws=ctypes.c_void_p(0x1000010)) == 10   # misaligned


@pytest.mark.parametrize("name,repack_image,repack_filter,order", [
    ("tiny_5x5_r3", "0", "0", None),      # the direct kernel reads both in place
    ("downsample_s2_n8_c64_56", "0", "0", "blocked"),
    ("pointwise_1x1_n32_c256_56", "0", "0", "blocked"),
    ("bottleneck_3x3_n32_c128_28", "0", "0", "blocked"),
    ("large_channel_n64_c512_14", "0", "0", "blocked"),
    ("dilated_asym_n16_c96_64x48", "1", "1", None),
])
def test_plans(name, repack_image, repack_filter, order):
    c = wl.case(name)
    a = _args(c)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation))
    assert f["repack_image"] == repack_image and f["repack_filter"] == repack_filter
    if order:
        assert f["order"] == order
    need = ci8.conv_fprop_i8_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation)
    assert (need == 0) == (repack_image == "0" and repack_filter == "0")
    if f["kernel"] == "direct":
        return
    # channel-innermost NHWC output -> lanes walk channels; NCHW -> pixels
    assert f["lanes"] == ("channels" if c.out.strides[1] == 1 else "pixels")


def test_footprint_offsets_fit_24_bits(monkeypatch):
    """The 3x3 footprint kernels form column offsets with a 24-bit product:
    a W stride of 2^23 bytes or more is planned on another kernel; image
    steps of any size across a launch's images are fine."""
    monkeypatch.setenv("CONV_I8_TILE", "f128x128")
    N, C, H, W, K = 2, 64, 9, 10, 40
    cl = wl.channels_last_strides((N, C, H, W))
    w = ci8.desc((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)), 1)
    y = ci8.desc((N, K, H, W), wl.channels_last_strides((N, K, H, W)), 2)

    def fields(strides):
        x = ci8.desc((N, C, H, W), strides, 1)
        return ci8.plan_fields(ci8.conv_fprop_i8_plan(x, w, y, 1, 1, 1, 1))

    dense = fields(cl)
    assert dense["tile"] == "f128x128" and dense["batch_chunk"] == "2"
    far = fields((1 << 24,) + tuple(cl[1:]))
    assert far["batch_chunk"] == "2" and far["tile"] == "f128x128"
    wide = fields((H * W << 23, 1, W << 23, 1 << 23))  # W stride 2^23 bytes
    assert wide["kernel"] != "footprint"


def _tuned_entries():
    path = os.path.join(os.path.dirname(os.path.abspath(ci8.__file__)), "csrc", "tuned_tiles.inc")
    rows = []
    for line in open(path):
        m = re.match(r"\{([-\d, ]+), \"([\w]+)\"\},", line.strip())
        if m:
            rows.append((tuple(int(v) for v in m.group(1).split(",")), m.group(2)))
    return rows


def test_tuned_tiles_are_planned(monkeypatch):
    """The measured tile table compiled into the library covers every
    workload, and the planner takes its tile (ahead of the cost model)."""
    monkeypatch.delenv("CONV_I8_TILE", raising=False)
    rows = dict(_tuned_entries())
    names = set(ci8.conv_i8_tile_names())
    assert set(rows.values()) <= names
    for name in wl.CASES:
        c = wl.case(name)
        a = _args(c)
        f = ci8.plan_fields(ci8.conv_fprop_i8_plan(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation))
        key = (0, *c.image.dims, c.filter.dims[0], *c.filter.dims[2:], *c.pre, *c.post, *c.stride,
               *c.dilation, 1 if f["lanes"] == "pixels" else 0)
        assert key in rows, name
        assert f["tile"] == rows[key], (name, f["tile"], rows[key])


def test_wgrad_tuned_tiles_are_planned(monkeypatch):
    """Weight-gradient rows of the table (keyed by the layer and dW's layout)
    give the tile of the gradient's one forward call; the split of its
    reduction stays the planner's.  A forced tile still wins."""
    monkeypatch.delenv("CONV_I8_TILE", raising=False)
    rows = {k: t for k, t in _tuned_entries() if k[0] == 1}
    assert rows, "no weight-gradient rows in the table"
    seen = 0
    for name in wl.CASES:
        c = wl.case(name)
        key = (1, *c.image.dims, c.filter.dims[0], *c.filter.dims[2:], *c.pre, *c.post, *c.stride,
               *c.dilation, 0 if c.filter.strides[1] == 1 else 1)
        if key not in rows:
            continue
        seen += 1
        x = ci8.desc(c.image.dims, c.image.strides, ci8.DT_INT8)
        dy = ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT8)
        dw = ci8.desc(c.filter.dims, c.filter.strides, ci8.DT_INT32)
        f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(x, dy, dw, c.pre, c.post, c.stride, c.dilation))
        assert f["tile"] == rows[key], (name, f["tile"], rows[key])
        assert int(f["workspace"]) == ci8.conv_wgrad_i8_workspace_size(x, dy, dw, c.pre, c.post, c.stride,
                                                                       c.dilation)
        other = "128x128x64" if rows[key] != "128x128x64" else "w256x128x64"
        monkeypatch.setenv("CONV_I8_TILE", other)
        f2 = ci8.plan_fields(ci8.conv_wgrad_i8_plan(x, dy, dw, c.pre, c.post, c.stride, c.dilation))
        monkeypatch.delenv("CONV_I8_TILE")
        assert f2["tile"] == other, (name, f2)
    assert seen == len(rows)


def _plan_raw(x, w, y, wptr, pre=(1, 1), post=(1, 1), st=(1, 1), dl=(1, 1)):
    pre_, post_, st_, dl_ = ci8._params(pre, post, st, dl, None)
    buf = ctypes.create_string_buffer(512)
    rc = ci8.lib.conv_fprop_i8_plan(ctypes.byref(x), None, ctypes.byref(w), wptr, ctypes.byref(y),
                                    pre_, post_, st_, dl_, buf, 512)
    assert rc == 0, ci8.STATUS[rc]
    return ci8.plan_fields(buf.value.decode())


def test_kmajor_filter_plans(monkeypatch):
    """A filter whose output channels are contiguous (an R, S, C, K filter, or
    the data gradient's view of a KRSC filter) is read in place by the 3x3
    tail tiles and by the im2col tiles of 64-channel stages over 64, 128 or
    256 columns (no repack, no filter workspace); a misaligned pointer, K not
    a multiple of 16, C not a multiple of 64 or another tile repack it."""
    monkeypatch.delenv("CONV_I8_TILE", raising=False)
    D = ci8.desc
    N, C, H, W, K = 8, 128, 14, 14, 96
    x = D((N, C, H, W), wl.channels_last_strides((N, C, H, W)), 1)
    y = D((N, K, H, W), wl.channels_last_strides((N, K, H, W)), 2)
    hwio = lambda k, c: D((k, c, 3, 3), (1, k, 3 * c * k, c * k), 1)       # [R][S][C][K] storage
    for tile in ("t256x128", "t128x128", "64x64x64", "128x128x64", "w256x128x64"):
        monkeypatch.setenv("CONV_I8_TILE", tile)
        f = _plan_raw(x, hwio(K, C), y, FAKE)
        assert (f["tile"], f["filter_read"], f["repack_filter"], f["workspace"]) == (tile, "kmajor", "0", "0"), f
        f = _plan_raw(x, hwio(K, C), y, ctypes.c_void_p(FAKE.value + 8))
        assert (f["filter_read"], f["repack_filter"]) == ("packed", "1") and int(f["workspace"]) > 0, f
        yk = D((N, 88, H, W), wl.channels_last_strides((N, 88, H, W)), 2)
        assert _plan_raw(x, hwio(88, C), yk, FAKE)["filter_read"] == "packed"
        x96 = D((N, 96, H, W), wl.channels_last_strides((N, 96, H, W)), 1)
        assert _plan_raw(x96, hwio(K, 96), y, FAKE)["filter_read"] == "packed"
    for tile in ("r256x128", "128x128x128", "w128x192x128"):
        monkeypatch.setenv("CONV_I8_TILE", tile)
        f = _plan_raw(x, hwio(K, C), y, FAKE)
        assert (f["tile"], f["filter_read"]) == (tile, "packed"), f
    # a channels-innermost filter stays read in place as before
    monkeypatch.setenv("CONV_I8_TILE", "t256x128")
    f = _plan_raw(x, D((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)), 1), y, FAKE)
    assert (f["filter_read"], f["repack_filter"]) == ("in_place", "0"), f


def test_wgrad_plan_arguments():
    D = ci8.desc
    x, dy = D((2, 3, 6, 7), (126, 42, 7, 1), 1), D((2, 4, 4, 5), (80, 20, 5, 1), 1)
    dw = D((4, 3, 3, 3), (27, 9, 3, 1), 2)
    pre, post, st, dl = ci8._params(0, 0, 1, 1, None)
    S = ci8.STATUS
    assert S[ci8.lib.conv_wgrad_i8_plan(ctypes.byref(x), None, ctypes.byref(dy), None, ctypes.byref(dw),
                                        pre, post, st, dl, 0, None, 64)] == "CONV_I8_ERR_NULL"
    f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(x, dy, dw))
    assert f["ksplit"] == "1" and "tile" in f
    bad = D((2, 4, 4, 6), (96, 24, 6, 1), 1)       # loss dims do not match the forward output
    with pytest.raises(ci8.ConvI8Error) as e:
        ci8.conv_wgrad_i8_plan(x, bad, dw)
    assert e.value.name == "CONV_I8_ERR_OUT_DIMS"
    assert ci8.conv_wgrad_i8_plan(x, D((2, 0, 4, 5), (0, 20, 5, 1), 1), D((0, 3, 3, 3), (27, 9, 3, 1), 2)) == "empty"


def test_tile_names():
    names = ci8.conv_i8_tile_names()
    assert len(names) == len(set(names)) and "t256x128" in names and "128x128x64" in names
    buf = ctypes.create_string_buffer(8)
    assert ci8.STATUS[ci8.lib.conv_i8_tile_names(buf, 8)] == "CONV_I8_ERR_PARAM"
    assert ci8.STATUS[ci8.lib.conv_i8_tile_names(None, 8)] == "CONV_I8_ERR_NULL"


def test_mfma_ceiling_argument_errors():
    S = ci8.STATUS
    assert S[ci8.lib.conv_i8_mfma_ceiling(4, 1, 1, None, None)] == "CONV_I8_ERR_NULL"
    assert S[ci8.lib.conv_i8_mfma_ceiling(0, 1, 1, FAKE, None)] == "CONV_I8_ERR_PARAM"
    assert S[ci8.lib.conv_i8_mfma_ceiling(4, 0, 1, FAKE, None)] == "CONV_I8_ERR_PARAM"
    assert S[ci8.lib.conv_i8_mfma_ceiling((1 << 20) + 1, 1, 1, FAKE, None)] == "CONV_I8_ERR_PARAM"


def test_direct_kernel_plans(monkeypatch):
    """Tiny problems whose operands need a repack run on the direct kernel
    (one launch, no workspace); a forced "direct" is refused above its size
    limit and the default tile runs instead."""
    monkeypatch.delenv("CONV_I8_TILE", raising=False)
    D = ci8.desc
    x, w = D((2, 3, 6, 7), (126, 42, 7, 1), 1), D((4, 3, 3, 3), (27, 9, 3, 1), 1)   # NCHW, KCRS
    y = D((2, 4, 4, 5), (80, 20, 5, 1), 2)
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(x, w, y))
    assert f["kernel"] == "direct" and f["workspace"] == "0" and f["repack_image"] == "0"
    assert ci8.conv_fprop_i8_workspace_size(x, w, y) == 0
    c = wl.case("large_channel_n64_c512_14")
    a = _args(c)
    monkeypatch.setenv("CONV_I8_TILE", "direct")
    f = ci8.plan_fields(ci8.conv_fprop_i8_plan(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation))
    assert f["tile"] == "128x128x64"


def test_empty_problems_are_ok_without_device_work():
    D = ci8.desc
    # N = 0: nothing to write, no pointers needed
    a = dict(x=D((0, 16, 5, 5), (400, 1, 80, 16), 1), w=D((4, 16, 3, 3), (144, 1, 48, 16), 1),
             y=D((0, 4, 3, 3), (36, 1, 12, 4), 2), pre=0, post=0, stride=1, dil=1)
    assert _call_ws(a, xp=None, wp=None, yp=None) == 0
    # K = 0
    a = dict(x=D((2, 16, 5, 5), (400, 1, 80, 16), 1), w=D((0, 16, 3, 3), (144, 1, 48, 16), 1),
             y=D((2, 0, 3, 3), (0, 1, 0, 0), 2), pre=0, post=0, stride=1, dil=1)
    assert _call_ws(a, xp=None, wp=None, yp=None) == 0


def test_window_larger_than_padded_image():
    D = ci8.desc
    x, w = D((1, 16, 2, 2), (64, 1, 32, 16), 1), D((1, 16, 3, 3), (144, 1, 48, 16), 1)
    with pytest.raises(ci8.ConvI8Error) as e:
        ci8.conv_fprop_i8_out_dims(x, w)
    assert e.value.name == "CONV_I8_ERR_OUT_DIMS"
    # C division would truncate (-1)/2 to 0 and claim one output row
    x = D((1, 16, 2, 5), (160, 1, 80, 16), 1)
    w = D((1, 16, 4, 3), (192, 1, 48, 16), 1)
    with pytest.raises(ci8.ConvI8Error):
        ci8.conv_fprop_i8_out_dims(x, w, stride=(2, 1))


def test_plan_cache_keys():
    """Plans are cached per problem; the cache must tell apart what changes a
    plan: a forced tile, the operands' alignment (in-place read or repack)
    and the problem itself."""
    c = wl.case("large_channel_n64_c512_14")
    dx = ci8.desc(c.image.dims, c.image.strides, 1)
    dw = ci8.desc(c.filter.dims, c.filter.strides, 1)
    dy = ci8.desc(c.out.dims, c.out.strides, 2)
    pre, post, st, dl = ci8._params(c.pre, c.post, c.stride, c.dilation, None)

    def plan(xp, wp, tile=None):
        old = os.environ.pop("CONV_I8_TILE", None)
        if tile:
            os.environ["CONV_I8_TILE"] = tile
        try:
            buf = ctypes.create_string_buffer(512)
            rc = ci8.lib.conv_fprop_i8_plan(ctypes.byref(dx), ctypes.c_void_p(xp), ctypes.byref(dw),
                                            ctypes.c_void_p(wp), ctypes.byref(dy), pre, post, st, dl, buf, 512)
            assert rc == 0
            return ci8.plan_fields(buf.value.decode())
        finally:
            os.environ.pop("CONV_I8_TILE", None)
            if old is not None:
                os.environ["CONV_I8_TILE"] = old

    base = plan(4096, 8192)
    assert plan(4096, 8192) == base                      # served from the cache
    assert base["repack_image"] == "0" and base["repack_filter"] == "0"
    assert plan(4096 + 8, 8192)["repack_image"] == "1"   # misaligned image: repacked
    assert plan(4096, 8192 + 4)["repack_filter"] == "1"
    assert plan(4096, 8192, "64x64x64")["tile"] == "64x64x64"
    assert plan(4096, 8192) == base
    # a different problem (one image fewer) is planned afresh
    dx2 = ci8.desc((63,) + tuple(c.image.dims[1:]), c.image.strides, 1)
    dy2 = ci8.desc((63,) + tuple(c.out.dims[1:]), c.out.strides, 2)
    buf = ctypes.create_string_buffer(512)
    assert ci8.lib.conv_fprop_i8_plan(ctypes.byref(dx2), ctypes.c_void_p(4096), ctypes.byref(dw),
                                      ctypes.c_void_p(8192), ctypes.byref(dy2), pre, post, st, dl, buf, 512) == 0
    assert ci8.plan_fields(buf.value.decode())["batch_chunk"] == "63"


def _call_rq(a, rq, ws_bytes=0, ws=None, xp=FAKE, wp=FAKE, yp=FAKE):
    p = ci8._params(a["pre"], a["post"], a["stride"], a["dil"], None)
    return ci8.lib.conv_fprop_i8_requant_ws(
        ctypes.byref(a["x"]), xp, ctypes.byref(a["w"]), wp, ctypes.byref(a["y"]), yp, *p,
        ctypes.byref(rq) if rq is not None else None, ws, ctypes.c_size_t(ws_bytes), None)


def test_requant_argument_errors():
    """The requantising entry wants an INT8 output and a sane parameter block,
    and checks both on the host before any device work."""
    c = wl.case("bottleneck_3x3_n32_c128_28")
    a8 = _args(c, y=ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT8))
    ok = ci8.Requant(None, 1.0, None, 0)
    assert _call_rq(_args(c), ok) == 2                                   # INT32 output: DTYPE
    assert _call_rq(a8, None) == 1                                       # no block: NULL
    assert _call_rq(a8, ci8.Requant(0x1000002, 1.0, None, 0)) == 5      # misaligned scale
    assert _call_rq(a8, ci8.Requant(None, 1.0, 0x1000001, 0)) == 5      # misaligned bias
    assert _call_rq(a8, ci8.Requant(None, float("nan"), None, 0)) == 5  # alpha must be finite
    assert _call_rq(a8, ci8.Requant(None, float("inf"), None, 1)) == 5
    # with a scale array alpha is unused
    bad_alpha = ci8.Requant(0x1000000, float("nan"), None, 0)
    assert _call_rq(a8, bad_alpha, yp=None) == 1                         # passes the block check
    need = ci8.conv_fprop_i8_requant_workspace_size(a8["x"], a8["w"], a8["y"], c.pre, c.post,
                                                    c.stride, c.dilation)
    assert need == ci8.conv_fprop_i8_workspace_size(_args(c)["x"], _args(c)["w"], _args(c)["y"],
                                                    c.pre, c.post, c.stride, c.dilation)
    with pytest.raises(ci8.ConvI8Error) as e:
        ci8.conv_fprop_i8_requant_workspace_size(a8["x"], a8["w"], _args(c)["y"], c.pre, c.post,
                                                 c.stride, c.dilation)
    assert e.value.name == "CONV_I8_ERR_DTYPE"


def test_requant_workspace_matches_plain():
    """Repacks do not depend on the output dtype."""
    c = wl.case("dilated_asym_n16_c96_64x48")
    a = _args(c)
    a8 = _args(c, y=ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT8))
    n32 = ci8.conv_fprop_i8_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation)
    n8 = ci8.conv_fprop_i8_requant_workspace_size(a8["x"], a8["w"], a8["y"], c.pre, c.post,
                                                  c.stride, c.dilation)
    assert n8 == n32 > 0
    assert _call_rq(a8, ci8.Requant(None, 1.0, None, 0), ws_bytes=n8 - 1, ws=FAKE) == 10


def _call_ex(a, mode, rq, ws_bytes=0, ws=None, xp=FAKE, wp=FAKE, yp=FAKE):
    p = ci8._params(a["pre"], a["post"], a["stride"], a["dil"], None)
    return ci8.lib.conv_fprop_i8_ex_ws(
        ctypes.byref(a["x"]), xp, ctypes.byref(a["w"]), wp, ctypes.byref(a["y"]), yp, *p, mode,
        ctypes.byref(rq) if rq is not None else None, ws, ctypes.c_size_t(ws_bytes), None)


def test_ex_entry_argument_errors():
    """The general entry: a known mode, INT32 output without a requantisation
    block, INT8 output with one; all checked on the host."""
    c = wl.case("bottleneck_3x3_n32_c128_28")
    a32 = _args(c)
    a8 = _args(c, y=ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT8))
    rq = ci8.Requant(None, 1.0, None, 0)
    assert _call_ex(a32, 2, None) == 5                    # unknown mode
    assert _call_ex(a32, -1, None) == 5
    assert _call_ex(a32, 0, rq) == 5                      # INT32 output with a block
    assert _call_ex(a8, 1, None) == 1                     # INT8 output without one
    a16 = _args(c, y=ci8.desc(c.out.dims, c.out.strides, 3))
    assert _call_ex(a16, 0, None) == 2                    # neither INT32 nor INT8
    # null output pointer is reported after the arguments check out
    assert _call_ex(a32, 1, None, yp=None) == 1
    for mode in (0, 1):
        for a in (a32, a8):
            n = ci8.conv_fprop_i8_ex_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post,
                                                    c.stride, c.dilation, mode=mode)
            assert n == 0
    c = wl.case("dilated_asym_n16_c96_64x48")
    a = _args(c)
    n0 = ci8.conv_fprop_i8_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride, c.dilation)
    n1 = ci8.conv_fprop_i8_ex_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride,
                                             c.dilation, mode=1)
    assert n1 == n0 > 0
    with pytest.raises(ci8.ConvI8Error) as e:
        ci8.conv_fprop_i8_ex_workspace_size(a["x"], a["w"], a["y"], c.pre, c.post, c.stride,
                                            c.dilation, mode=3)
    assert e.value.name == "CONV_I8_ERR_PARAM"


def _dgrad_args(N=2, K=8, C=16, H=9, W=7, R=3, S=3, pre=(1, 1), post=(1, 1), st=(2, 2), dl=(1, 1)):
    D = ci8.desc
    P = (H + pre[0] + post[0] - dl[0] * (R - 1) - 1) // st[0] + 1
    Q = (W + pre[1] + post[1] - dl[1] * (S - 1) - 1) // st[1] + 1
    dy = D((N, K, P, Q), (K * P * Q, 1, Q * K, K), ci8.DT_INT8)
    w = D((K, C, R, S), (C * R * S, 1, S * C, C), ci8.DT_INT8)
    dx = D((N, C, H, W), (C * H * W, 1, W * C, C), ci8.DT_INT32)
    return dy, w, dx, pre, post, st, dl


def _call_dgrad(dy, w, dx, pre, post, st, dl, mode=0, ws_bytes=0, ws=None, yp=FAKE):
    p = ci8._params(pre, post, st, dl, None)
    return ci8.lib.conv_dgrad_i8_ws(ctypes.byref(dy), FAKE, ctypes.byref(w), FAKE, ctypes.byref(dx),
                                    yp, *p, mode, ws, ctypes.c_size_t(ws_bytes), None)


def test_dgrad_argument_errors():
    dy, w, dx, pre, post, st, dl = _dgrad_args()
    D = ci8.desc
    # dx INT8 or dy INT32: dtype
    assert _call_dgrad(dy, w, D(dx.dims, dx.strides, ci8.DT_INT8), pre, post, st, dl) == 2
    assert _call_dgrad(D(dy.dims, dy.strides, ci8.DT_INT32), w, dx, pre, post, st, dl) == 2
    # dY's spatial size must be the forward output size of dX's
    bad = D((2, 8, 4, 4), (128, 1, 32, 8), ci8.DT_INT8)
    assert _call_dgrad(bad, w, dx, pre, post, st, dl) == 7
    # channel mismatch between filter and dX
    assert _call_dgrad(dy, w, D((2, 12, 9, 7), (756, 1, 84, 12), ci8.DT_INT32), pre, post, st, dl) == 6
    # K*R*S beyond the exact range
    a = _dgrad_args(K=15000, C=16)
    assert _call_dgrad(*a) == 9
    # unknown mode, overlapping dX
    assert _call_dgrad(dy, w, dx, pre, post, st, dl, mode=2) == 5
    assert _call_dgrad(dy, w, D(dx.dims, (0, 1, 7, 1), ci8.DT_INT32), pre, post, st, dl) == 8
    # null dX pointer once everything else is right
    assert _call_dgrad(dy, w, dx, pre, post, st, dl, yp=None) == 1


@pytest.mark.parametrize("st,dl", [((1, 1), (1, 1)), ((2, 2), (1, 1)), ((2, 3), (2, 1)), ((4, 4), (2, 2))])
def test_dgrad_workspace(st, dl):
    """One forward call per stride phase; above the direct kernel's size the
    transposed filter always needs a repack, so the workspace is at least the
    packed filter."""
    dy, w, dx, pre, post, _, _ = _dgrad_args(K=32, C=64, st=st, dl=dl)
    n = ci8.conv_dgrad_i8_workspace_size(dy, w, dx, pre, post, st, dl)
    assert n >= 64 * 32 * 9 // max(1, st[0] * st[1])
    assert _call_dgrad(dy, w, dx, pre, post, st, dl, ws_bytes=n - 1, ws=FAKE) == 10


def test_wgrad_argument_errors():
    D = ci8.desc
    dy, w, dx, pre, post, st, dl = _dgrad_args()
    x = D(dx.dims, dx.strides, ci8.DT_INT8)        # the image
    dw = D(w.dims, w.strides, ci8.DT_INT32)        # the filter gradient

    def call(x_, dy_, dw_, mode=0, yp=FAKE, ws_bytes=0, ws=None, stv=st):
        p = ci8._params(pre, post, stv, dl, None)
        return ci8.lib.conv_wgrad_i8_ws(ctypes.byref(x_), FAKE, ctypes.byref(dy_), FAKE,
                                        ctypes.byref(dw_), yp, *p, mode, ws, ctypes.c_size_t(ws_bytes), None)
    assert call(x, dy, D(dw.dims, dw.strides, ci8.DT_INT8)) == 2          # dW must be INT32
    assert call(D(x.dims, x.strides, ci8.DT_INT32), dy, dw) == 2
    assert call(x, D((2, 8, 4, 4), (128, 1, 32, 8), ci8.DT_INT8), dw) == 7  # dY not the output size
    assert call(x, dy, D((8, 12, 3, 3), (108, 1, 36, 12), ci8.DT_INT32)) == 6
    assert call(x, dy, dw, mode=5) == 5
    assert call(x, dy, D(dw.dims, (0, 1, 0, 0), ci8.DT_INT32)) == 8        # overlapping dW
    assert call(x, dy, dw, yp=None) == 1
    # N*P*Q beyond the exact range: 600 images of 15x15 outputs
    big_x = D((600, 16, 15, 15), (3600, 1, 240, 16), ci8.DT_INT8)
    big_dy = D((600, 8, 15, 15), (1800, 1, 120, 8), ci8.DT_INT8)
    assert call(big_x, big_dy, dw, stv=(1, 1)) == 9
    # a tiny problem: the direct kernel reads the transposed operands in place
    assert ci8.conv_wgrad_i8_workspace_size(x, dy, dw, pre, post, st, dl) == 0
    dy, w, dx, pre, post, st, dl = _dgrad_args(K=32, C=64)
    N, C, H, W = dx.dims
    x = D(dx.dims, (C * H * W, H * W, W, 1), ci8.DT_INT8)   # NCHW: not read in place
    dw = D(w.dims, w.strides, ci8.DT_INT32)
    n = ci8.conv_wgrad_i8_workspace_size(x, dy, dw, pre, post, st, dl)
    assert n > 0                                 # both transposed operands are repacked
    assert call(x, dy, dw, ws_bytes=n - 1, ws=FAKE) == 10
    # channels-last, many pixels: read in place, the pixels split into partial copies of dW
    dy, w, dx, pre, post, st, dl = _dgrad_args(N=8, K=32, C=64, H=40, W=40)
    x = D(dx.dims, dx.strides, ci8.DT_INT8)
    dw = D(w.dims, w.strides, ci8.DT_INT32)
    f = ci8.plan_fields(ci8.conv_wgrad_i8_plan(x, dy, dw, pre, post, st, dl))
    n = ci8.conv_wgrad_i8_workspace_size(x, dy, dw, pre, post, st, dl)
    assert f["kernel"] == "wgrad_in_place" and int(f["ksplit"]) > 1, f
    assert n == int(f["workspace"]) == int(f["ksplit"]) * 32 * 64 * 9 * 4
    assert call(x, dy, dw, ws_bytes=n - 1, ws=FAKE) == 10


def test_wgrad_in_place_plans(monkeypatch):
    """Which weight gradients the in-place kernel takes: channels-last image
    and loss with C and K multiples of 16 and a dense dW; anything else, or a
    forced tile, goes to the forward call of the transposed operands.  A dW
    of more tile-taps (128x128 per filter tap) than half the CUs is split for
    two workgroups per CU."""
    monkeypatch.delenv("CONV_I8_TILE", raising=False)
    D = ci8.desc

    def plan(N=4, K=64, C=64, H=20, W=20, R=3, S=3, x_nchw=False, dw_gaps=False, st=(1, 1), pad=(1, 1)):
        dy, w, dx, pre, post, st_, dl = _dgrad_args(N=N, K=K, C=C, H=H, W=W, R=R, S=S, pre=pad, post=pad, st=st)
        xs = (C * H * W, H * W, W, 1) if x_nchw else dx.strides
        ws_ = (R * S * 2 * C, 1, S * 2 * C, 2 * C) if dw_gaps else w.strides
        return ci8.plan_fields(ci8.conv_wgrad_i8_plan(D(dx.dims, xs, ci8.DT_INT8), dy,
                                                      D(w.dims, ws_, ci8.DT_INT32), pre, post, st_, dl))
    f = plan()
    assert (f["kernel"], f["image_rows"]) == ("wgrad_in_place", "per_tap"), f
    f = plan(R=1, S=1, pad=(0, 0))
    assert (f["kernel"], f["image_rows"]) == ("wgrad_in_place", "linear"), f
    f = plan(R=1, S=1, pad=(0, 0), st=(2, 2))
    assert (f["kernel"], f["image_rows"]) == ("wgrad_in_place", "per_tap"), f
    assert plan(x_nchw=True)["kernel"] != "wgrad_in_place"
    assert plan(C=40)["kernel"] != "wgrad_in_place"
    assert plan(dw_gaps=True)["kernel"] != "wgrad_in_place"
    f = plan(N=64, K=512, C=512, H=14, W=14)       # the large-channel layer: 144 tile-taps
    assert (f["kernel"], f["tiles"], f["ksplit"]) == ("wgrad_in_place", "144", "3"), f
    f = plan(N=64, K=256, C=256, H=14, W=14)       # 36 tile-taps: one workgroup per CU
    assert (f["kernel"], f["tiles"], f["ksplit"]) == ("wgrad_in_place", "36", "7"), f
    monkeypatch.setenv("CONV_I8_TILE", "128x128x64")
    assert plan()["tile"] == "128x128x64"


class _NoCalls:
    """Stands in for the loaded library: any use of an entry fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"the wrapper reached the C entry {name}")


def _cpu_case():
    x = torch.zeros((1, 16, 5, 5), dtype=torch.int8)
    w = torch.zeros((4, 16, 3, 3), dtype=torch.int8)
    y = torch.zeros((1, 4, 3, 3), dtype=torch.int32)
    return x, w, y


@pytest.mark.parametrize("call", [
    lambda x, w, y: ci8.conv_fprop_i8(x, w, y),
    lambda x, w, y: ci8.conv_fprop_i8(x, w),
    lambda x, w, y: ci8.conv_fprop_i8_ws(x, w, y, None),
    lambda x, w, y: ci8.conv_fprop_i8_plain(x, w, y),
    lambda x, w, y: ci8.conv_fprop_i8_requant(x, w),
    lambda x, w, y: ci8.conv_fprop_i8_requant_ws(x, w, y.to(torch.int8), None),
    lambda x, w, y: ci8.conv_fprop_i8_requant_plain(x, w, y.to(torch.int8)),
    lambda x, w, y: ci8.conv_fprop_i8_ex_ws(x, w, y, None),
    lambda x, w, y: ci8.conv_fprop_i8_mode(x, w, ci8.MODE_CONVOLUTION),
    lambda x, w, y: ci8.conv_dgrad_i8(y.to(torch.int8), w, torch.zeros((1, 16, 5, 5), dtype=torch.int32)),
    lambda x, w, y: ci8.conv_dgrad_i8_ws(y.to(torch.int8), w, torch.zeros((1, 16, 5, 5), dtype=torch.int32), None),
    lambda x, w, y: ci8.conv_dgrad_i8_plain(y.to(torch.int8), w, torch.zeros((1, 16, 5, 5), dtype=torch.int32)),
    lambda x, w, y: ci8.conv_wgrad_i8(x, y.to(torch.int8), torch.zeros((4, 16, 3, 3), dtype=torch.int32)),
    lambda x, w, y: ci8.conv_wgrad_i8_ws(x, y.to(torch.int8), torch.zeros((4, 16, 3, 3), dtype=torch.int32), None),
    lambda x, w, y: ci8.conv_wgrad_i8_plain(x, y.to(torch.int8), torch.zeros((4, 16, 3, 3), dtype=torch.int32)),
])
def test_wrappers_refuse_host_tensors_before_any_c_call(monkeypatch, call):
    """Host tensors would hand host pointers to the kernels: every wrapper
    refuses them before it reaches the library."""
    x, w, y = _cpu_case()
    monkeypatch.setattr(ci8, "lib", _NoCalls())
    with pytest.raises(ValueError, match="expected a GPU tensor"):
        call(x, w, y)


def test_wrappers_refuse_non_tensors(monkeypatch):
    x, w, y = _cpu_case()
    monkeypatch.setattr(ci8, "lib", _NoCalls())
    with pytest.raises(TypeError, match="expected a torch.Tensor"):
        ci8.conv_fprop_i8_ws(x.numpy(), w, y, None)
