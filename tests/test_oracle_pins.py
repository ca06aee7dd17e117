"""Pins of the CPU oracle against references other than itself (CPU only)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import build as obuild

from . import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def _golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def test_printed_shapes(orc):
    pins.check_printed_shapes(orc, _golden("printed_shapes.json")["cases"])


def test_case_table_out_dims(orc):
    # the literal output dims of every workload agree with the oracle's rule
    for c in wl.CASES.values():
        assert orc.out_dims(c.image.dims, c.filter.dims, c.pre, c.post, c.stride, c.dilation) == c.out.dims


def test_out_dims_errors(orc):
    with pytest.raises(oracle.OracleError) as e:   # window larger than padded image
        orc.out_dims((1, 1, 2, 2), (1, 1, 3, 3), 0, 0, 1, 1)
    assert e.value.code == 2
    with pytest.raises(oracle.OracleError) as e:   # channel mismatch
        orc.out_dims((1, 2, 5, 5), (1, 3, 3, 3), 0, 0, 1, 1)
    assert e.value.code == 2
    for bad in [dict(stride=0), dict(dil=0), dict(pre=-1), dict(post=(0, -1))]:
        a = dict(pre=0, post=0, stride=1, dil=1)
        a.update(bad)
        with pytest.raises(oracle.OracleError) as e:
            orc.out_dims((1, 1, 5, 5), (1, 1, 3, 3), a["pre"], a["post"], a["stride"], a["dil"])
        assert e.value.code == 1
    # the numerator is checked before dividing: -1 // 2 would floor to -1,
    # C division would truncate to 0 and wrongly give one output row
    with pytest.raises(oracle.OracleError):
        orc.out_dims((1, 1, 2, 5), (1, 1, 4, 3), 0, 0, (2, 1), 1)


def test_random_vs_brute_force(orc):
    pins.check_random_vs_brute_force(orc, n_cases=1500, seed=1)


def test_one_dim_sweep(orc):
    pins.check_one_dim_sweep(orc)


def test_forum_answer_shape_brute_force(orc):
    # "Building a From-Scratch INT8 Strided Convolution Kernel", "Correctness
    # Testing": 1x3x32x32 input, 64x3x3x3 kernel, stride 1 -> 1x64x30x30,
    # compared for exact equality.
    rng = np.random.default_rng(2)
    x = pins.rand_i8(rng, (1, 3, 32, 32))
    w = pins.rand_i8(rng, (64, 3, 3, 3))
    y = orc.conv_fprop(x, w)
    assert tuple(y.shape) == (1, 64, 30, 30)
    assert np.array_equal(y.numpy(), pins.brute_force(x.numpy(), w.numpy(), (0, 0), (0, 0), (1, 1), (1, 1)))


@pytest.mark.parametrize("check", [pins.check_offcentre_delta, pins.check_identity_1x1,
                                   pins.check_ones_count, pins.check_constant_min,
                                   pins.check_layouts, pins.check_metamorphic, pins.check_points])
def test_closed_forms_and_invariants(orc, check):
    check(orc)


def test_forum_output_decode():
    """The forum's wrong cuDNN output is the true result saturated to int8 and
    read back as int32: the library must refuse an INT8 output and write INT32.
    (Pins the reading that the output dtype is INT32 and never saturates.)"""
    g = _golden("forum_5x5_r3.json")
    truth = np.array(g["torch_conv2d_int32"], dtype=np.int64).reshape(-1)
    # every value lies within the bound 9 taps * 128 * 128
    assert np.abs(truth).max() <= 9 * 128 * 128
    sat = np.clip(truth, -128, 127).astype(np.int8)
    buf = np.zeros(9 * 4, dtype=np.uint8)          # the zero-filled int32 output
    buf[:9] = sat.view(np.uint8)
    as_i32 = buf.view("<i4").reshape(3, 3)
    assert as_i32.tolist() == g["cudnn_output_int32"]


def test_requant_forum_bytes(orc):
    """The requantising epilogue at scale 1 reproduces the bytes of the forum's
    INT8 cuDNN output from its torch results."""
    pins.check_requant_forum_bytes(orc, _golden("forum_5x5_r3.json"))


def test_requant_exact(orc):
    pins.check_requant_exact(orc)


def test_requant_nonfinite(orc):
    pins.check_requant_nonfinite(orc)


def test_requant_conv(orc):
    pins.check_requant_conv(orc)


def test_convolution_mode(orc):
    pins.check_convolution_mode(orc)


def test_dgrad(orc):
    pins.check_dgrad(orc)


def test_wgrad(orc):
    pins.check_wgrad(orc)


@pytest.mark.parametrize("name", wl.CASE_ORDER)
def test_workloads_vs_f64_library_conv(orc, name):
    """Oracle == float64 torch conv2d on every workload at full size."""
    c = wl.case(name)
    d = wl.make_inputs(c, c.seed_base)
    y = orc.conv_fprop(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation)
    ref = pins.f64_library_conv(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation)
    assert torch.equal(y.to(torch.int64), ref)


def test_worst_case_closed_forms(orc):
    """Dilated asymmetric workload: the constant -128 quarter equals
    16384 * C * T(p, q); the mixed quarters equal -128 times a window sum."""
    c = wl.case("dilated_asym_n16_c96_64x48")
    d = wl.make_inputs(c, c.seed_base)
    x, w = d["x"], d["w"]
    N, C, H, W = c.image.dims
    K, _, R, S = c.filter.dims
    _, _, P, Q = c.out.dims
    T = pins.in_bounds_taps(H, W, R, S, c.pre, c.stride, c.dilation, P, Q)
    rng = np.random.default_rng(0)
    pts = np.stack([rng.integers(0, N, 400), rng.integers(0, K, 400),
                    rng.integers(0, P, 400), rng.integers(0, Q, 400)], axis=1)
    pts[:100, 0] = rng.integers(N // 2, N, 100)
    pts[:100, 1] = rng.integers(K // 2, K, 100)
    vals = orc.conv_fprop_points(x, w, pts, c.pre, c.post, c.stride, c.dilation)
    xn, wn = x.numpy().astype(np.int64), w.numpy().astype(np.int64)
    for (n, k, p, q), v in zip(pts, vals):
        taps = [(r, s) for r in range(R) for s in range(S)
                if 0 <= p * c.stride[0] - c.pre[0] + r * c.dilation[0] < H
                and 0 <= q * c.stride[1] - c.pre[1] + s * c.dilation[1] < W]
        if n >= N // 2 and k >= K // 2:
            assert v == 16384 * C * T[p, q]
        elif n >= N // 2:
            assert v == -128 * sum(int(wn[k, :, r, s].sum()) for r, s in taps)
        elif k >= K // 2:
            assert v == -128 * sum(int(xn[n, :, p * c.stride[0] - c.pre[0] + r * c.dilation[0],
                                               q * c.stride[1] - c.pre[1] + s * c.dilation[1]].sum())
                                   for r, s in taps)
    # interior maximum: every tap inside
    assert vals.max() <= 16384 * C * R * S
    assert 16384 * C * R * S == 23592960


def test_overflow_is_reported(orc):
    # C*R*S = 135000 > 131071 products of 16384 can leave int32
    x = torch.full((1, 15000, 3, 3), -128, dtype=torch.int8)
    w = torch.full((1, 15000, 3, 3), -128, dtype=torch.int8)
    with pytest.raises(oracle.OracleError) as e:
        orc.conv_fprop(x, w)
    assert e.value.code == 4


MUTATIONS = [
    # (description, original text, replacement)
    ("padding test dropped", "if (h < 0 || h >= H || wc < 0 || wc >= Wd)", "if (h < 0 || wc < 0)"),
    ("pre-padding sign flipped", "p * stride[0] - pre[0]", "p * stride[0] + pre[0]"),
    ("column pre-padding ignored", "q * stride[1] - pre[1]", "q * stride[1]"),
    ("row dilation dropped", "r * dil[0];", "r;"),
    ("column stride dropped", "q * stride[1] - pre[1] + s * dil[1]", "q - pre[1] + s * dil[1]"),
    ("filter taps transposed", "fr * ws[2] + fs * ws[3]", "fs * ws[2] + fr * ws[3]"),
    ("filter read with the channel stride twice", "k * ws[0] + c * ws[1]", "k * ws[1] + c * ws[1]"),
    ("image h/w strides swapped", "h * xs[2] + wc * xs[3]", "h * xs[3] + wc * xs[2]"),
    ("filter flipped in cross-correlation", "fr = mode ? R - 1 - r : r;", "fr = R - 1 - r;"),
    ("convolution mode flips rows only", "fs = mode ? S - 1 - s : s;", "fs = s;"),
    ("convolution mode flips nothing", "fr = mode ? R - 1 - r : r;", "fr = r;"),
    ("dgrad ignores the stride divisibility", "pn % stride[0] != 0 || ", ""),
    ("dgrad pre-padding sign", "h + pre[0] - r * dil[0]", "h - pre[0] - r * dil[0]"),
    ("dgrad column dilation dropped", "x + pre[1] - s * dil[1]", "x + pre[1] - s"),
    ("dgrad last row of dY dropped", "pn / stride[0] >= P", "pn / stride[0] >= P - 1"),
    ("wgrad row stride dropped", "const int64_t h = p * stride[0] - pre[0] + r * dil[0];\n                            if (h < 0 || h >= H)", "const int64_t h = p - pre[0] + r * dil[0];\n                            if (h < 0 || h >= H)"),
    ("wgrad ignores the image's right edge", "if (wc < 0 || wc >= W)\n                                    continue;\n                                acc += (int64_t)dy", "if (wc < 0)\n                                    continue;\n                                acc += (int64_t)dy"),
    ("wgrad mode ignored", "const int64_t gr = mode ? R - 1 - r : r, gs", "const int64_t gr = r, gs"),
    ("dgrad mode ignored", "const int64_t fs = mode ? S - 1 - s : s;\n                acc", "const int64_t fs = s;\n                acc"),
    ("unsigned widening of int8", "const int64_t xv = x[", "const int64_t xv = (uint8_t)x["),
    ("last channel dropped", "for (int64_t c = 0; c < C; ++c)", "for (int64_t c = 0; c + 1 < C; ++c)"),
    ("first filter row dropped", "for (int64_t r = 0; r < R; ++r)", "for (int64_t r = 1; r < R; ++r)"),
    ("output size off by one", "return span / stride + 1;", "return span / stride;"),
    ("output size ignores post padding", "in + pre + post - dil", "in + pre - dil"),
    ("output written transposed", "p * ystr[2] + q * ystr[3]", "q * ystr[2] + p * ystr[3]"),
    ("saturating int8 store", "(int32_t)(uint32_t)(uint64_t)acc", "(int32_t)(acc > 127 ? 127 : acc < -128 ? -128 : acc)"),
    ("requant truncates", "v = nearbyintf(v);", "v = truncf(v);"),
    ("requant rounds half away from zero", "v = nearbyintf(v);", "v = roundf(v);"),
    ("requant multiplies then adds", "fmaf((float)acc, s, b)", "((float)acc * s + b)"),
    ("requant ReLU dropped", "if (relu && v < 0.0f)", "if (0 && relu && v < 0.0f)"),
    ("requant clamps at -127", "if (v < -128.0f)\n        v = -128.0f;", "if (v < -127.0f)\n        v = -127.0f;"),
    ("requant per-tensor scale", "const float s = scale ? scale[k] : alpha;", "const float s = scale ? scale[0] : alpha;"),
    ("requant bias ignored", "const float b = bias ? bias[k] : 0.0f;", "const float b = 0.0f;"),
    ("requant channel from the wrong index", "scale ? scale[ch[i]] : alpha", "scale ? scale[i % 2] : alpha"),
    ("requant NaN written as -128", "v = 0.0f;  /* NaN", "v = -128.0f;  /* NaN"),
]


@pytest.mark.slow
def test_mutants_are_caught(tmp_path):
    """Each plausible mistake planted in a copy of the oracle fails a pin."""
    src = open(obuild.SRC).read()
    script = os.path.join(HERE, "mutant_check.py")
    # the unmutated copy passes
    lib = obuild.compile_oracle(obuild.SRC, str(tmp_path / "base.so"))
    r = subprocess.run([sys.executable, script, lib], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    survivors = []
    for i, (desc, old, new) in enumerate(MUTATIONS):
        assert src.count(old) >= 1, f"mutation anchor not found: {old}"
        cfile = tmp_path / f"m{i}.c"
        cfile.write_text(src.replace(old, new))
        lib = obuild.compile_oracle(str(cfile), str(tmp_path / f"m{i}.so"), extra=("-w",))
        r = subprocess.run([sys.executable, script, lib], capture_output=True, text=True, timeout=300)
        if r.returncode == 0:
            survivors.append(desc)
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_empty_operands(orc):
    """C = 0 sums nothing and H = 0 leaves only padding: all outputs are 0,
    as brute force gives."""
    x = torch.empty((2, 0, 5, 5), dtype=torch.int8)
    w = torch.empty((3, 0, 3, 3), dtype=torch.int8)
    y = orc.conv_fprop(x, w, 1, 1)
    assert tuple(y.shape) == (2, 3, 5, 5) and (y == 0).all()
    x = torch.empty((2, 4, 0, 3), dtype=torch.int8)
    w = torch.ones((3, 4, 1, 2), dtype=torch.int8)
    y = orc.conv_fprop(x, w, (1, 0), (2, 1))
    ref = pins.brute_force(x.numpy(), w.numpy(), (1, 0), (2, 1), (1, 1), (1, 1))
    assert tuple(y.shape) == ref.shape == (2, 3, 3, 3) and (y == 0).all()
