"""The allocation-free entry conv_fprop_i8_noalloc (static per-GPU scratch
array) against conv_fprop_i8_ws with a caller workspace: byte-identical
outputs on two calls in a row, the second on a smaller problem, and a
problem too large for the array refused before any device work."""
import ctypes

import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


def _dev():
    return torch.device("cuda:0")


def _pair(ci8, c, seed):
    """(x, w, out via the _ws entry, out via the noalloc entry) for a case."""
    d = wl.make_inputs(c, seed)
    xg = wl.to_device(d["x_storage"], c.image, _dev())[1]
    wg = wl.to_device(d["w_storage"], c.filter, _dev())[1]
    need = ci8.conv_fprop_i8_workspace_size(xg, wg, ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT32),
                                            c.pre, c.post, c.stride, c.dilation)
    assert 0 < need <= ci8.NOALLOC_SCRATCH_BYTES, need
    ys = wl.alloc_output(c.out, _dev())[1]
    yn = wl.alloc_output(c.out, _dev(), fill=-12345)[1]
    ws = torch.empty(need, dtype=torch.uint8, device=_dev())
    print(f"[gpu] noalloc vs ws: {c.name} seed {seed} workspace {need} bytes", flush=True)
    ci8.conv_fprop_i8_ws(xg, wg, ys, ws, c.pre, c.post, c.stride, c.dilation)
    ci8.conv_fprop_i8_noalloc(xg, wg, yn, c.pre, c.post, c.stride, c.dilation)
    torch.cuda.synchronize()
    return d, ys.cpu(), yn.cpu()


def test_noalloc_matches_workspace_entry(ci8):
    # first call: the dilated case (both operands repacked, ~5 MB of scratch)
    big = wl.case("dilated_asym_n16_c96_64x48")
    d, ys, yn = _pair(ci8, big, big.seed_base)
    assert torch.equal(ys, yn)
    # second call, smaller problem: the same layer on two images (smaller
    # repacks into the same array, which still holds the first call's bytes)
    small = wl.ConvCase(name="dilated_n2", image=wl.TensorSpec((2, 96, 64, 48), big.image.strides,
                                                               storage=2 * 96 * 64 * 96),
                        filter=big.filter, out=wl.TensorSpec((2, 192, 32, 44), wl.contiguous_strides((2, 192, 32, 44))),
                        pre=big.pre, post=big.post, stride=big.stride, dilation=big.dilation,
                        recipe=big.recipe, seed_base=big.seed_base + 1)
    d2, ys2, yn2 = _pair(ci8, small, small.seed_base)
    assert torch.equal(ys2, yn2)
    ref = oracle.conv_fprop(d2["x"], d2["w"], small.pre, small.post, small.stride, small.dilation)
    assert torch.equal(yn2, ref)
    # and the first problem again after the smaller one
    d3, ys3, yn3 = _pair(ci8, big, big.seed_base + 2)
    assert torch.equal(ys3, yn3)


def test_noalloc_refuses_problems_beyond_its_scratch(ci8):
    """An NCHW image of 25.7 MB must be repacked into more than the array
    holds: refused with CONV_I8_ERR_SCRATCH, output untouched."""
    N, C, H, W, K = 256, 512, 14, 14, 16
    x = torch.zeros((N, C, H, W), dtype=torch.int8, device=_dev())
    w = torch.zeros((K, C, 3, 3), dtype=torch.int8, device=_dev())
    y = torch.full((N, K, H, W), 7, dtype=torch.int32, device=_dev())
    need = ci8.conv_fprop_i8_workspace_size(x, w, y, 1, 1, 1, 1)
    assert need > ci8.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ci8.ConvI8Error) as e:
        ci8.conv_fprop_i8_noalloc(x, w, y, 1, 1, 1, 1)
    assert e.value.name == "CONV_I8_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert bool((y == 7).all())


def test_noalloc_without_workspace(ci8):
    """Problems that need no workspace (operands read in place: the tiny
    layer on the direct kernel, the large-channel layer on the 3x3 kernel)
    go through the allocation-free entry unchanged."""
    for name in ("tiny_5x5_r3", "large_channel_n64_c512_14"):
        c = wl.case(name)
        d = wl.make_inputs(c, c.seed_base + 3)
        xg = wl.to_device(d["x_storage"], c.image, _dev())[1]
        wg = wl.to_device(d["w_storage"], c.filter, _dev())[1]
        assert ci8.conv_fprop_i8_workspace_size(xg, wg, ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT32),
                                                c.pre, c.post, c.stride, c.dilation) == 0
        yn = wl.alloc_output(c.out, _dev(), fill=-7)[1]
        print(f"[gpu] noalloc without workspace: {name}", flush=True)
        ci8.conv_fprop_i8_noalloc(xg, wg, yn, c.pre, c.post, c.stride, c.dilation)
        torch.cuda.synchronize()
        ref = oracle.conv_fprop(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation)
        assert torch.equal(yn.cpu(), ref), name
