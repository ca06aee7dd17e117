"""HIP graph capture of the workspace entries (the allocation-free,
synchronisation-free calls): replays must give the eager bytes, also with
eager work and synchronisations between the replays."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ci8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int8_convolution_forward_amd as m
    return m


@pytest.mark.parametrize("name", ["tiny_5x5_r3", "downsample_s2_n8_c64_56",
                                  "dilated_asym_n16_c96_64x48", "pointwise_1x1_n32_c256_56"])
@pytest.mark.parametrize("epilogue", ["int32", "requant"])
def test_graph_replay_matches_eager(ci8, name, epilogue):
    c = wl.case(name)
    dev = torch.device("cuda:0")
    d = wl.make_inputs(c, c.seed_base)
    x = wl.to_device(d["x_storage"], c.image, dev)[1]
    w = wl.to_device(d["w_storage"], c.filter, dev)[1]
    K = c.filter.dims[0]
    rq = epilogue == "requant"
    scale = (torch.rand(K, generator=torch.Generator().manual_seed(3)) * 1e-3).to(dev) if rq else None
    bias = (torch.rand(K, generator=torch.Generator().manual_seed(4)) * 10 - 5).to(dev) if rq else None
    dt = torch.int8 if rq else torch.int32
    buf = torch.empty(c.out.storage_size, dtype=dt, device=dev)
    out = torch.as_strided(buf, c.out.dims, c.out.strides, c.out.offset)
    size = (ci8.conv_fprop_i8_requant_workspace_size if rq else ci8.conv_fprop_i8_workspace_size)(
        x, w, out, c.pre, c.post, c.stride, c.dilation)
    ws = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
    args = (c.pre, c.post, c.stride, c.dilation)

    def call():
        if rq:
            ci8.conv_fprop_i8_requant_ws(x, w, out, ws if size else None, scale, 1.0, bias, True, *args)
        else:
            ci8.conv_fprop_i8_ws(x, w, out, ws if size else None, *args)

    print(f"[gpu] graph {name} {epilogue} workspace={size}", flush=True)
    buf.fill_(7)
    call()
    torch.cuda.synchronize()
    eager = buf.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the plan cache off the capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        buf.fill_(i + 11)                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf, eager), f"replay {i} differs from the eager call"


def _replays_match(call, buf, view):
    """Eager result first, then three replays of a captured call, with eager
    work and synchronisations between them (refilling the whole buffer);
    every replay must give the eager result in every element of the output
    view (the gaps of a strided view keep the fill)."""
    buf.fill_(7)
    call()
    torch.cuda.synchronize()
    eager = view.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the plan cache off the capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        buf.fill_(i + 11)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(view, eager), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("name,mode", [("downsample_s2_n8_c64_56", 0), ("bottleneck_3x3_n32_c128_28", 0),
                                       ("dilated_asym_n16_c96_64x48", 1)])
def test_graph_replay_dgrad(ci8, name, mode):
    """The data gradient under capture: the phase filters' repack and one
    forward launch per stride phase (four phases for the stride-2 layer)."""
    c = wl.case(name)
    dev = torch.device("cuda:0")
    d = wl.make_inputs(c, c.seed_base + 2)
    w = wl.to_device(d["w_storage"], c.filter, dev)[1]
    g = torch.Generator().manual_seed(17)
    dy_buf = torch.randint(-128, 128, (c.out.storage_size,), dtype=torch.int8, generator=g).to(dev)
    dy = torch.as_strided(dy_buf, c.out.dims, c.out.strides)
    dx_strides = wl.channels_last_strides(c.image.dims)
    buf = torch.empty(wl.TensorSpec(c.image.dims, dx_strides).storage_size, dtype=torch.int32, device=dev)
    dx = torch.as_strided(buf, c.image.dims, dx_strides)
    args = (c.pre, c.post, c.stride, c.dilation)
    size = ci8.conv_dgrad_i8_workspace_size(dy, w, dx, *args, mode=mode)
    ws = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
    print(f"[gpu] graph dgrad {name} mode={mode} workspace={size}", flush=True)
    _replays_match(lambda: ci8.conv_dgrad_i8_ws(dy, w, dx, ws if size else None, *args, mode=mode), buf, dx)


@pytest.mark.parametrize("name,layout", [("bottleneck_3x3_n32_c128_28", "dense"),
                                         ("bottleneck_3x3_n32_c128_28", "gaps"),
                                         ("downsample_s2_n8_c64_56", "dense"),
                                         ("dilated_asym_n16_c96_64x48", "dense")])
def test_graph_replay_wgrad(ci8, name, layout):
    """The weight gradient under capture: the transposed operands' repacks
    and one forward launch, including the split reduction (partial copies
    plus their sum for a dense dW, zeros plus atomic adds for a dW with gaps
    between its pixels)."""
    c = wl.case(name)
    dev = torch.device("cuda:0")
    d = wl.make_inputs(c, c.seed_base + 3)
    x = wl.to_device(d["x_storage"], c.image, dev)[1]
    g = torch.Generator().manual_seed(19)
    dy_buf = torch.randint(-128, 128, (c.out.storage_size,), dtype=torch.int8, generator=g).to(dev)
    dy = torch.as_strided(dy_buf, c.out.dims, c.out.strides)
    K, C, R, S = c.filter.dims
    if layout == "dense":
        dws = wl.TensorSpec(c.filter.dims, c.filter.strides)
    else:
        dws = wl.TensorSpec((K, C, R, S), (R * S * 2 * C, 1, S * 2 * C, 2 * C))
    buf = torch.empty(dws.storage_size, dtype=torch.int32, device=dev)
    dw = torch.as_strided(buf, dws.dims, dws.strides, dws.offset)
    args = (c.pre, c.post, c.stride, c.dilation)
    size = ci8.conv_wgrad_i8_workspace_size(x, dy, dw, *args)
    ws = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
    print(f"[gpu] graph wgrad {name} {layout} workspace={size}", flush=True)
    _replays_match(lambda: ci8.conv_wgrad_i8_ws(x, dy, dw, ws if size else None, *args), buf, dw)

