"""GPU parity of the data gradient (conv_dgrad_i8) against the oracle's
dgrad (pinned to float64 autograd and the adjoint identity): bit-exact over
the whole dX buffer, guard bands included."""
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


def run_dgrad_check(ci8, dy_storage, dyspec, w_storage, wspec, dxspec, pre, post, st, dl, mode=0,
                    label="", entry="ws"):
    dy_cpu = torch.as_strided(dy_storage, dyspec.dims, dyspec.strides, dyspec.offset)
    w_cpu = torch.as_strided(w_storage, wspec.dims, wspec.strides, wspec.offset)
    dyg = wl.to_device(dy_storage, dyspec, _dev())[1]
    wg = wl.to_device(w_storage, wspec, _dev())[1]
    size = dxspec.storage_size + 2 * GUARD
    buf = torch.full((size,), wl.SENTINEL, dtype=torch.int32, device=_dev())
    dxg = torch.as_strided(buf, dxspec.dims, dxspec.strides, dxspec.offset + GUARD)
    print(f"[gpu] dgrad {label} dy={dyspec.dims}/{dyspec.strides} w={wspec.dims}/{wspec.strides} "
          f"dx={dxspec.dims}/{dxspec.strides} pre={pre} post={post} stride={st} dil={dl} "
          f"mode={mode} entry={entry}", flush=True)
    if entry == "ws":
        ci8.conv_dgrad_i8(dyg, wg, dxg, pre, post, st, dl, mode=mode)
    else:
        ci8.conv_dgrad_i8_plain(dyg, wg, dxg, pre, post, st, dl, mode=mode)
    torch.cuda.synchronize()
    got = buf.cpu()
    ref = torch.full((size,), wl.SENTINEL, dtype=torch.int32)
    rv = torch.as_strided(ref, dxspec.dims, dxspec.strides, dxspec.offset + GUARD)
    oracle.conv_dgrad(dy_cpu, w_cpu, None, pre, post, st, dl, out=rv, mode=mode)
    if not torch.equal(got, ref):
        diff = (got != ref).nonzero().reshape(-1)
        raise AssertionError(f"{label}: {diff.numel()} elements differ, first at {diff[:5].tolist()}: "
                             f"got {got[diff[:5]].tolist()} want {ref[diff[:5]].tolist()}")


def _rand_storage(spec, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(-128, 128, (spec.storage_size,), dtype=torch.int8, generator=g)


@pytest.mark.parametrize("name", wl.CASE_ORDER)
@pytest.mark.parametrize("mode", [0, 1])
def test_workload_dgrad(ci8, name, mode):
    """The data gradient of every workload: dY in the forward output's layout,
    the workload's filter, dX in the image's logical dims (channels_last)."""
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base + 3)
    dyspec = wl.TensorSpec(c.out.dims, c.out.strides)
    dxspec = wl.TensorSpec(c.image.dims, wl.channels_last_strides(c.image.dims))
    run_dgrad_check(ci8, _rand_storage(dyspec, 5 + mode), dyspec, d["w_storage"], c.filter, dxspec,
                    c.pre, c.post, c.stride, c.dilation, mode=mode, label=name)


def test_random_dgrad_problems(ci8):
    """Strides up to 4 (phases with no taps), dilation, padding larger than the
    filter reach (cropped dY rows), non-square filters, NCHW and NHWC."""
    rng = np.random.default_rng(43)
    done = 0
    while done < 40:
        N, K, C = int(rng.integers(1, 4)), int(rng.integers(1, 70)), int(rng.integers(1, 70))
        H, W = (int(v) for v in rng.integers(1, 20, 2))
        R, S = (int(v) for v in rng.integers(1, 6, 2))
        pre = tuple(int(v) for v in rng.integers(0, 5, 2))
        post = tuple(int(v) for v in rng.integers(0, 5, 2))
        st = tuple(int(v) for v in rng.integers(1, 5, 2))
        dl = tuple(int(v) for v in rng.integers(1, 4, 2))
        try:
            od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        except oracle.OracleError:
            continue
        lay = lambda d: (wl.channels_last_strides(d) if rng.integers(0, 2) else wl.contiguous_strides(d))
        dyspec = wl.TensorSpec(od, lay(od))
        wspec = wl.TensorSpec((K, C, R, S), lay((K, C, R, S)))
        dxspec = wl.TensorSpec((N, C, H, W), lay((N, C, H, W)))
        run_dgrad_check(ci8, _rand_storage(dyspec, 100 + done), dyspec, _rand_storage(wspec, 200 + done),
                        wspec, dxspec, pre, post, st, dl, mode=done % 2, label=f"random {done}",
                        entry="plain" if done % 5 == 0 else "ws")
        done += 1


def test_random_dgrad_kmajor_problems(ci8, capfd, monkeypatch):
    """Random layers whose filter views the kernels read k-major (KRSC or
    R, S, C, K filters, K a multiple of 64, C a multiple of 16) with a
    channels-last loss: strides 1-3 (one launch for up to four phases),
    dilation, padding past the taps' reach, non-square filters, both modes;
    the k-major reads and the one-launch path must both occur."""
    rng = np.random.default_rng(97)
    monkeypatch.setenv("CONV_I8_LOG", "1")
    done = 0
    while done < 30:
        N, K, C = int(rng.integers(1, 4)), 64 * int(rng.integers(1, 3)), 16 * int(rng.integers(1, 7))
        H, W = (int(v) for v in rng.integers(3, 18, 2))
        R, S = (int(v) for v in rng.integers(1, 5, 2))
        pre = tuple(int(v) for v in rng.integers(0, 4, 2))
        post = tuple(int(v) for v in rng.integers(0, 4, 2))
        st = tuple(int(v) for v in rng.integers(1, 4, 2))
        dl = tuple(int(v) for v in rng.integers(1, 3, 2))
        try:
            od = oracle.out_dims((N, C, H, W), (K, C, R, S), pre, post, st, dl)
        except oracle.OracleError:
            continue
        dyspec = wl.TensorSpec(od, wl.channels_last_strides(od))
        wstr = wl.channels_last_strides((K, C, R, S)) if done % 2 else (1, K, S * C * K, C * K)
        wspec = wl.TensorSpec((K, C, R, S), wstr)
        dxspec = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
        run_dgrad_check(ci8, _rand_storage(dyspec, 300 + done), dyspec, _rand_storage(wspec, 400 + done),
                        wspec, dxspec, pre, post, st, dl, mode=(done // 2) % 2, label=f"random k-major {done}",
                        entry="plain" if done % 7 == 0 else "ws")
        done += 1
    logged = capfd.readouterr().err
    assert "filter_read=kmajor" in logged
    assert "data-gradient phases in one launch" in logged


@pytest.mark.parametrize("dy_layout", ["nhwc", "nchw"])
@pytest.mark.parametrize("mode", [0, 1])
def test_dgrad_phase_filters_read_kmajor(ci8, monkeypatch, capfd, dy_layout, mode):
    """A stride-2 layer (the downsample workload: 4 phases, 64 input channels
    per phase): every phase reads its view of the KRSC filter in place,
    k-major, so no filter is packed; a channels-last loss is read in place, an
    NCHW one packed once for all phases; either way the four phases run in
    one launch.  Bit-exact."""
    c = wl.case("downsample_s2_n8_c64_56")
    d = wl.make_inputs(c, c.seed_base + 8)
    dims = c.out.dims
    strides = wl.channels_last_strides(dims) if dy_layout == "nhwc" else wl.contiguous_strides(dims)
    dyspec = wl.TensorSpec(dims, strides)
    dxspec = wl.TensorSpec(c.image.dims, wl.channels_last_strides(c.image.dims))
    monkeypatch.setenv("CONV_I8_LOG", "1")
    run_dgrad_check(ci8, _rand_storage(dyspec, 31 + mode), dyspec, d["w_storage"], c.filter, dxspec,
                    c.pre, c.post, c.stride, c.dilation, mode=mode, label=f"k-major {dy_layout}")
    logged = capfd.readouterr().err
    plans = [ci8.plan_fields(l) for l in logged.splitlines() if "repack_filter=" in l]
    assert len(plans) == 4, logged
    assert all(p["repack_filter"] == "0" and p["filter_read"] == "kmajor" for p in plans), logged
    assert all(p["repack_image"] == "0" for p in plans), logged
    assert ("loss packed once for 4 phases" in logged) == (dy_layout == "nchw"), logged
    assert "4 data-gradient phases in one launch" in logged, logged


@pytest.mark.parametrize("dy_layout,loss_in_place", [("nhwc", True), ("nchw", False)])
@pytest.mark.parametrize("mode", [0, 1])
def test_dgrad_phase_filters_packed_once(ci8, monkeypatch, capfd, dy_layout, loss_in_place, mode):
    """A stride-2 layer with 48 output channels (4 phases whose 48 input
    channels are no whole 64-channel stage, so no phase reads its filter view
    k-major): every phase's filter view is packed by one repack launch before
    the phases (which also packs an NCHW loss once for all of them), so each
    phase plan reads its loss and its filter in place.  Bit-exact."""
    N, C, H, W, K = 4, 64, 20, 20, 48
    pre, post, st, dl = (1, 1), (1, 1), (2, 2), (1, 1)
    wspec = wl.TensorSpec((K, C, 3, 3), wl.channels_last_strides((K, C, 3, 3)))
    dims = oracle.out_dims((N, C, H, W), (K, C, 3, 3), pre, post, st, dl)
    strides = wl.channels_last_strides(dims) if dy_layout == "nhwc" else wl.contiguous_strides(dims)
    dyspec = wl.TensorSpec(dims, strides)
    dxspec = wl.TensorSpec((N, C, H, W), wl.channels_last_strides((N, C, H, W)))
    monkeypatch.setenv("CONV_I8_LOG", "1")
    run_dgrad_check(ci8, _rand_storage(dyspec, 31 + mode), dyspec, _rand_storage(wspec, 41 + mode), wspec, dxspec,
                    pre, post, st, dl, mode=mode, label=f"packed {dy_layout}")
    logged = capfd.readouterr().err
    plans = [ci8.plan_fields(l) for l in logged.splitlines() if "repack_filter=" in l]
    assert len(plans) == 4, logged
    assert all(p["repack_filter"] == "0" and p["repack_image"] == "0" for p in plans), logged
    assert not any(p["filter_read"] == "kmajor" for p in plans), logged
    assert ("loss packed once" in logged) == (not loss_in_place), logged
