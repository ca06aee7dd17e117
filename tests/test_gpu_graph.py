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
