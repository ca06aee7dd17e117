"""Independent references that pin the oracle (CPU only).

Nothing here imports the HIP library.  Each check takes an ``oracle.Oracle``
object so that the mutation test can run the same checks against deliberately
broken builds of the oracle.

* ``brute_force`` computes the convolution a second, unrelated way: explicit
  zero padding of the image (``numpy.pad``), zero insertion between filter taps
  for dilation, then a dot product of every stride-spaced window with the
  dilated filter.  Where the oracle evaluates bounds per tap, this one never
  tests a bound.
* ``f64_library_conv`` is torch's CPU conv2d in float64 after an explicit
  asymmetric ``F.pad`` — exact here, since every partial sum is an integer far
  below 2**53 (the forum page checks its INT8 result against torch's conv2d).
* the closed forms (delta filters, ones-by-ones counts, constant operands) come
  from the definition on the cuDNN "Convolutions" page, section
  "Convolution Fprop", worked out by hand.
* true convolution (mode 1) is checked against ``scipy.signal.convolve2d``,
  the textbook 2-D convolution (it flips the kernel), summed over channels,
  with padding by ``numpy.pad``, dilation by zero insertion and stride by
  subsampling; and against the brute force above fed the filter reversed
  along both spatial axes.
* the data gradient (dgrad) is checked against float64 autograd of torch's
  conv2d with respect to the image (exact for these integer sums), and by the
  adjoint identity <fprop(X, W), dY> = <X, dgrad(dY, W)> in int64 against
  the pinned forward oracle, in both modes.
* the weight gradient (wgrad) likewise: float64 autograd with respect to the
  filter, and <fprop(X, W), dY> = <W, wgrad(X, dY)> in int64.
* ``exact_requant`` evaluates the requantising INT8 epilogue with exact
  rational arithmetic (``fractions.Fraction``): the fused multiply-add is the
  exact value ``acc*s + b`` rounded once to the nearest binary32 (ties to an
  even significand, found by comparing the neighbouring binary32 values
  exactly), then ReLU, Python's ``round`` (half to even) and the clamp to
  [-128, 127] of the INT8 store in "Building a From-Scratch INT8 Strided
  Convolution Kernel", step 2.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F


def brute_force(x: np.ndarray, w: np.ndarray, pre, post, stride, dil) -> np.ndarray:
    """int64 conv by explicit padding, zero-inserted dilation and windows."""
    x = np.asarray(x, dtype=np.int64)
    w = np.asarray(w, dtype=np.int64)
    N, C, H, W = x.shape
    K, C2, R, S = w.shape
    assert C == C2
    xp = np.pad(x, ((0, 0), (0, 0), (pre[0], post[0]), (pre[1], post[1])))
    Rd, Sd = dil[0] * (R - 1) + 1, dil[1] * (S - 1) + 1
    wd = np.zeros((K, C, Rd, Sd), dtype=np.int64)
    wd[:, :, ::dil[0], ::dil[1]] = w
    Hp, Wp = xp.shape[2], xp.shape[3]
    if Hp < Rd or Wp < Sd:
        return np.zeros((N, K, 0, 0), dtype=np.int64)
    P = len(range(0, Hp - Rd + 1, stride[0]))
    Q = len(range(0, Wp - Sd + 1, stride[1]))
    y = np.zeros((N, K, P, Q), dtype=np.int64)
    wflat = wd.reshape(K, -1)
    for p in range(P):
        for q in range(Q):
            win = xp[:, :, p * stride[0]:p * stride[0] + Rd, q * stride[1]:q * stride[1] + Sd]
            y[:, :, p, q] = win.reshape(N, -1) @ wflat.T
    return y


def f64_library_conv(x: torch.Tensor, w: torch.Tensor, pre, post, stride, dil) -> torch.Tensor:
    xp = F.pad(x.to(torch.float64), (pre[1], post[1], pre[0], post[0]))
    y = F.conv2d(xp, w.to(torch.float64), stride=tuple(stride), dilation=tuple(dil))
    return y.round().to(torch.int64)


def in_bounds_taps(H, W, R, S, pre, stride, dil, P, Q) -> np.ndarray:
    """T[p, q] = number of filter taps (r, s) that land inside the image."""
    rows = np.array([sum(1 for r in range(R) if 0 <= p * stride[0] - pre[0] + r * dil[0] < H)
                     for p in range(P)], dtype=np.int64)
    cols = np.array([sum(1 for s in range(S) if 0 <= q * stride[1] - pre[1] + s * dil[1] < W)
                     for q in range(Q)], dtype=np.int64)
    return rows[:, None] * cols[None, :]


def rand_i8(rng: np.random.Generator, shape) -> torch.Tensor:
    return torch.from_numpy(rng.integers(-128, 128, size=shape, dtype=np.int64).astype(np.int8))


# --------------------------------------------------------------------------
# Check routines (raise AssertionError on the first disagreement).
# --------------------------------------------------------------------------

def check_random_vs_brute_force(orc, n_cases: int = 300, seed: int = 7) -> None:
    """Random small problems over the full parameter grid vs brute force."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < n_cases:
        N, C, K = (int(v) for v in rng.integers(1, 4, size=3))
        H, W = (int(v) for v in rng.integers(1, 8, size=2))
        R, S = (int(v) for v in rng.integers(1, 4, size=2))
        st = tuple(int(v) for v in rng.integers(1, 4, size=2))
        dl = tuple(int(v) for v in rng.integers(1, 4, size=2))
        pre = tuple(int(v) for v in rng.integers(0, 3, size=2))
        post = tuple(int(v) for v in rng.integers(0, 3, size=2))
        if H + pre[0] + post[0] - dl[0] * (R - 1) - 1 < 0 or W + pre[1] + post[1] - dl[1] * (S - 1) - 1 < 0:
            continue
        x = rand_i8(rng, (N, C, H, W))
        w = rand_i8(rng, (K, C, R, S))
        y = orc.conv_fprop(x, w, pre, post, st, dl)
        ref = brute_force(x.numpy(), w.numpy(), pre, post, st, dl)
        assert tuple(y.shape) == ref.shape, (y.shape, ref.shape, (N, C, H, W, K, R, S, st, dl, pre, post))
        assert np.array_equal(y.numpy().astype(np.int64), ref), (N, C, H, W, K, R, S, st, dl, pre, post)
        done += 1


def check_one_dim_sweep(orc, seed: int = 11) -> None:
    """Every (H, R, stride, dilation, pre, post) with H<=7, R<=3, the rest <=2/3,
    in the row direction and, transposed, in the column direction."""
    rng = np.random.default_rng(seed)
    for H in range(1, 8):
        for R in range(1, 4):
            for st in range(1, 4):
                for dl in range(1, 4):
                    for pre in range(0, 3):
                        for post in range(0, 3):
                            if H + pre + post - dl * (R - 1) - 1 < 0:
                                continue
                            for axis in (0, 1):
                                if axis == 0:
                                    xs, ws = (1, 2, H, 2), (2, 2, R, 2)
                                    a = dict(pre=(pre, 1), post=(post, 0), stride=(st, 1), dil=(dl, 1))
                                else:
                                    xs, ws = (1, 2, 2, H), (2, 2, 2, R)
                                    a = dict(pre=(1, pre), post=(0, post), stride=(1, st), dil=(1, dl))
                                x = rand_i8(rng, xs)
                                w = rand_i8(rng, ws)
                                y = orc.conv_fprop(x, w, **a)
                                ref = brute_force(x.numpy(), w.numpy(), a["pre"], a["post"],
                                                  a["stride"], a["dil"])
                                assert np.array_equal(y.numpy().astype(np.int64), ref), (H, R, st, dl, pre, post, axis)


def check_offcentre_delta(orc) -> None:
    """Filter = 1 at one off-centre tap (r0, s0) on the diagonal k == c:
    Y[n,k,p,q] = X[n,k, p*sh - ph + r0*dh, q*sw - pw + s0*dw] (0 outside)."""
    rng = np.random.default_rng(3)
    for (R, S, r0, s0, st, dl, pre, post) in [
            (3, 5, 0, 3, (1, 1), (1, 1), (1, 2), (2, 1)),
            (3, 5, 2, 1, (2, 1), (2, 2), (2, 1), (1, 3)),
            (2, 3, 1, 0, (1, 2), (3, 1), (0, 2), (1, 0))]:
        C = 3
        x = rand_i8(rng, (2, C, 9, 8))
        w = torch.zeros((C, C, R, S), dtype=torch.int8)
        for k in range(C):
            w[k, k, r0, s0] = 1
        y = orc.conv_fprop(x, w, pre, post, st, dl).numpy()
        N, K, P, Q = y.shape
        xn = x.numpy().astype(np.int64)
        for p in range(P):
            for q in range(Q):
                h = p * st[0] - pre[0] + r0 * dl[0]
                ww = q * st[1] - pre[1] + s0 * dl[1]
                want = xn[:, :, h, ww] if (0 <= h < 9 and 0 <= ww < 8) else np.zeros((N, K), np.int64)
                assert np.array_equal(y[:, :, p, q], want), (R, S, r0, s0, p, q)


def check_identity_1x1(orc) -> None:
    """1x1 delta filter (W[k,c] = [k == c]) reproduces X, subsamples it under
    a stride, and embeds it in zeros under padding."""
    rng = np.random.default_rng(5)
    x = rand_i8(rng, (2, 4, 7, 6))
    w = torch.eye(4, dtype=torch.int8).reshape(4, 4, 1, 1)
    y = orc.conv_fprop(x, w)
    assert torch.equal(y, x.to(torch.int32))
    y = orc.conv_fprop(x, w, stride=(2, 3))
    assert torch.equal(y, x[:, :, ::2, ::3].to(torch.int32))
    y = orc.conv_fprop(x, w, pre=(1, 2), post=(2, 0))
    z = torch.zeros((2, 4, 10, 8), dtype=torch.int32)
    z[:, :, 1:8, 2:8] = x.to(torch.int32)
    assert torch.equal(y, z)


def check_ones_count(orc) -> None:
    """All-ones image and filter: every output equals C * (in-bounds taps);
    C*R*S wherever the whole window is inside."""
    for (C, H, W, R, S, pre, post, st, dl) in [
            (5, 6, 7, 3, 3, (0, 0), (0, 0), (1, 1), (1, 1)),
            (3, 9, 8, 3, 5, (2, 1), (1, 3), (2, 1), (2, 2)),
            (2, 5, 5, 2, 3, (1, 1), (1, 1), (1, 2), (1, 1))]:
        x = torch.ones((2, C, H, W), dtype=torch.int8)
        w = torch.ones((3, C, R, S), dtype=torch.int8)
        y = orc.conv_fprop(x, w, pre, post, st, dl).numpy()
        _, _, P, Q = y.shape
        T = in_bounds_taps(H, W, R, S, pre, st, dl, P, Q)
        assert np.array_equal(y, np.broadcast_to(C * T, y.shape)), (C, H, W, R, S)
        if pre == (0, 0) and post == (0, 0):
            assert (y == C * R * S).all()


def check_constant_min(orc) -> None:
    """Image and filter constant -128: each in-bounds tap adds 16384 per channel."""
    C, H, W, R, S = 4, 9, 8, 3, 5
    pre, post, st, dl = (2, 1), (1, 3), (2, 1), (2, 2)
    x = torch.full((1, C, H, W), -128, dtype=torch.int8)
    w = torch.full((2, C, R, S), -128, dtype=torch.int8)
    y = orc.conv_fprop(x, w, pre, post, st, dl).numpy()
    T = in_bounds_taps(H, W, R, S, pre, st, dl, y.shape[2], y.shape[3])
    assert np.array_equal(y[0, 0], 16384 * C * T)


def check_layouts(orc) -> None:
    """Same logical values as NCHW, NHWC, a 2x-wide strided view, a permuted
    filter and a zero-stride broadcast image give identical outputs."""
    rng = np.random.default_rng(9)
    x = rand_i8(rng, (2, 5, 7, 6))
    w = rand_i8(rng, (3, 5, 3, 2))
    a = dict(pre=(1, 0), post=(0, 2), stride=(2, 1), dil=(1, 2))
    ref = orc.conv_fprop(x, w, **a)
    nhwc = x.contiguous(memory_format=torch.channels_last)
    assert torch.equal(orc.conv_fprop(nhwc, w.contiguous(memory_format=torch.channels_last), **a), ref)
    wide = torch.zeros((2, 5, 7, 12), dtype=torch.int8)
    wide[..., ::2] = x
    wide[..., 1::2] = rand_i8(rng, (2, 5, 7, 6))
    assert torch.equal(orc.conv_fprop(wide[..., ::2], w, **a), ref)
    krsc_view = w.permute(0, 2, 3, 1).contiguous().permute(0, 3, 1, 2)
    assert torch.equal(orc.conv_fprop(x, krsc_view, **a), ref)
    row = rand_i8(rng, (1, 5, 7, 6))
    bcast = row.expand(4, 5, 7, 6)
    y = orc.conv_fprop(bcast, w, **a)
    y1 = orc.conv_fprop(row, w, **a)
    assert all(torch.equal(y[i], y1[0]) for i in range(4))
    # output written through strides lands in the right places
    out_cl = torch.full(ref.shape, -1, dtype=torch.int32).contiguous(memory_format=torch.channels_last)
    orc.conv_fprop(x, w, out=out_cl, **a)
    assert torch.equal(out_cl, ref)


def check_metamorphic(orc) -> None:
    """Stride = subsampled stride-1 output; dilation = zero-inserted filter;
    padding = explicit zero pad; linearity in X and W; slicing N and K."""
    rng = np.random.default_rng(13)
    x = rand_i8(rng, (3, 4, 11, 10))
    w = rand_i8(rng, (5, 4, 3, 2))
    base = orc.conv_fprop(x, w, pre=(1, 2), post=(1, 0))
    strided = orc.conv_fprop(x, w, pre=(1, 2), post=(1, 0), stride=(3, 2))
    assert torch.equal(strided, base[:, :, ::3, ::2])
    # dilation (2, 3) == dilation 1 with a zero-inserted filter
    wz = torch.zeros((5, 4, 5, 4), dtype=torch.int8)
    wz[:, :, ::2, ::3] = w
    assert torch.equal(orc.conv_fprop(x, w, dil=(2, 3)), orc.conv_fprop(x, wz))
    # padding == explicit zero pad, then no padding
    xp = F.pad(x, (2, 1, 1, 3))
    assert torch.equal(orc.conv_fprop(x, w, pre=(1, 2), post=(3, 1)), orc.conv_fprop(xp, w))
    # linearity (values kept small so sums stay int8)
    xa = torch.from_numpy(rng.integers(-64, 64, size=(3, 4, 11, 10)).astype(np.int8))
    xb = torch.from_numpy(rng.integers(-64, 64, size=(3, 4, 11, 10)).astype(np.int8))
    ya, yb, yab = (orc.conv_fprop(v, w) for v in (xa, xb, xa + xb))
    assert torch.equal(yab, ya + yb)
    wa = torch.from_numpy(rng.integers(-64, 64, size=(5, 4, 3, 2)).astype(np.int8))
    wb = torch.from_numpy(rng.integers(-64, 64, size=(5, 4, 3, 2)).astype(np.int8))
    assert torch.equal(orc.conv_fprop(x, wa + wb), orc.conv_fprop(x, wa) + orc.conv_fprop(x, wb))
    # negation of X negates Y (catches an unsigned widening of int8)
    xn = torch.from_numpy(rng.integers(-127, 128, size=(3, 4, 11, 10)).astype(np.int8))
    assert torch.equal(orc.conv_fprop(-xn, w), -orc.conv_fprop(xn, w))
    # slicing the batch or the filters slices the output
    assert torch.equal(orc.conv_fprop(x[1:], w), orc.conv_fprop(x, w)[1:])
    assert torch.equal(orc.conv_fprop(x, w[2:4]), orc.conv_fprop(x, w)[:, 2:4])


def check_printed_shapes(orc, cases) -> None:
    for c in cases:
        got = orc.out_dims(c["image"], c["filter"], c["pre"], c["post"], c["stride"], c["dilation"])
        assert list(got) == c["out"], (c, got)


def check_points(orc) -> None:
    """The per-element entry agrees with the full one."""
    rng = np.random.default_rng(17)
    x = rand_i8(rng, (2, 3, 9, 8))
    w = rand_i8(rng, (4, 3, 3, 5))
    a = dict(pre=(2, 1), post=(1, 3), stride=(2, 1), dil=(2, 2))
    y = orc.conv_fprop(x, w, **a).numpy()
    idx = np.array([[n, k, p, q] for n in range(2) for k in range(4)
                    for p in range(y.shape[2]) for q in range(y.shape[3])], dtype=np.int64)
    v = orc.conv_fprop_points(x, w, idx, **a)
    assert np.array_equal(v, y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].astype(np.int64))


def _f32_nearest(fr: Fraction) -> np.float32:
    """The binary32 value nearest to the exact rational ``fr``, ties to an
    even significand (no overflow: |fr| stays far below 2**127 here)."""
    if fr == 0:
        return np.float32(0.0)
    c = np.float32(float(fr))              # within one ulp of the answer
    cands = {float(c), float(np.nextafter(c, np.float32(np.inf))),
             float(np.nextafter(c, np.float32(-np.inf)))}

    def key(v):
        odd = int(np.array(v, dtype=np.float32).view(np.uint32)) & 1
        return (abs(Fraction(v) - fr), odd)
    return np.float32(min(cands, key=key))


def exact_requant(acc: int, s: float, b: float, relu: bool) -> int:
    """INT8 epilogue of one exact sum: binary32(acc) * s + b rounded once,
    ReLU, round half to even, saturate."""
    a = _f32_nearest(Fraction(int(acc)))   # the sum as a binary32 value
    v = _f32_nearest(Fraction(float(a)) * Fraction(float(np.float32(s))) +
                     Fraction(float(np.float32(b))))
    v = float(v)
    if relu and v < 0:
        v = 0.0
    r = round(v)                           # half to even
    return max(-128, min(127, r))


def check_requant_forum_bytes(orc, golden) -> None:
    """Scale 1, no bias, no ReLU is the saturating INT8 store: the forum's
    torch results become exactly the bytes its INT8 cuDNN output held."""
    truth = np.array(golden["torch_conv2d_int32"], dtype=np.int64).reshape(-1)
    got = orc.requant_values(truth, 0)
    buf = np.zeros(len(truth) * 4, dtype=np.uint8)
    buf[:len(truth)] = got.view(np.uint8)
    assert buf.view("<i4").reshape(3, 3).tolist() == golden["cudnn_output_int32"]


def _muladd_differs_cases(n: int = 200000, seed: int = 23):
    """(acc, s, b) where one rounding (fused) and two roundings (multiply,
    then add) give different INT8 results: acc*s lies just above some k+1/2
    but rounds to it as binary32, and b = -floor(.) cancels the integer part.
    All values are exact in float64 (acc < 2**17, s has 24 bits)."""
    rng = np.random.default_rng(seed)
    acc = rng.integers(1000, 1 << 17, n).astype(np.float64)
    s = rng.uniform(0.25, 4.0, n).astype(np.float32).astype(np.float64)
    p = acc * s                                   # exact
    p32 = p.astype(np.float32).astype(np.float64)
    hit = (p32 - np.floor(p32) == 0.5) & (p > p32)
    b = -np.floor(p32[hit])
    return acc[hit].astype(np.int64), s[hit].astype(np.float32), b.astype(np.float32)


def check_requant_exact(orc) -> None:
    """The epilogue equals the exact rational evaluation on ties, large sums
    (beyond 2**24, where binary32 rounds the sum), cancellations that tell a
    fused multiply-add from a multiply then an add, and random values; also
    the ReLU identity and per-channel indexing."""
    rng = np.random.default_rng(29)
    accs, scales, biases = [], [], []
    # exact ties k + 1/2 (scale 1/2, 1/4): half to even
    t = np.arange(-301, 302, dtype=np.int64)
    accs += [t, t]
    scales += [np.full(t.size, 0.5, np.float32), np.full(t.size, 0.25, np.float32)]
    biases += [np.zeros(t.size, np.float32), np.zeros(t.size, np.float32)]
    # large sums: binary32 rounds them; tiny scales bring them into range
    big = np.concatenate([rng.integers(1 << 24, (1 << 31) - 1, 300),
                          -rng.integers(1 << 24, 1 << 31, 300),
                          np.array([(1 << 24) + 1, (1 << 24) + 3, (1 << 25) + 2, 2147483647,
                                    -2147483648])]).astype(np.int64)
    accs.append(big)
    scales.append((2.0 ** rng.integers(-26, -18, big.size)).astype(np.float32))
    biases.append(rng.uniform(-3, 3, big.size).astype(np.float32))
    # fused vs unfused
    a, s_, b = _muladd_differs_cases()
    assert a.size >= 20, "search found too few cancellation cases"
    accs.append(a[:200])
    scales.append(s_[:200])
    biases.append(b[:200])
    # random
    r = rng.integers(-(1 << 27), 1 << 27, 2000).astype(np.int64)
    accs.append(r)
    scales.append((rng.choice([-1, 1], r.size) * 2.0 ** rng.uniform(-24, 0, r.size)).astype(np.float32))
    biases.append(rng.uniform(-300, 300, r.size).astype(np.float32))
    acc = np.concatenate(accs)
    sc = np.concatenate(scales)
    bi = np.concatenate(biases)
    ch = np.arange(acc.size, dtype=np.int64)     # one channel per value: per-channel lookup
    for relu in (False, True):
        got = orc.requant_values(acc, ch, scale=sc, bias=bi, relu=relu)
        want = np.array([exact_requant(int(x), float(y), float(z), relu)
                         for x, y, z in zip(acc, sc, bi)], dtype=np.int8)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (relu, [(int(acc[i]), float(sc[i]), float(bi[i]), int(got[i]),
                                       int(want[i])) for i in bad[:5]])
        if relu:
            assert np.array_equal(got, np.maximum(orc.requant_values(acc, ch, scale=sc, bias=bi), 0))
    # alpha applies to every channel when there is no scale array
    got = orc.requant_values(t, 0, alpha=0.5)
    assert np.array_equal(got, np.array([exact_requant(int(x), 0.5, 0.0, False) for x in t], np.int8))


def check_requant_nonfinite(orc) -> None:
    """Non-finite scale or bias: the pages are silent; the reading taken is
    that a NaN after the multiply-add is written as 0 and an infinity
    saturates.  Expected values written out by hand from that rule (IEEE:
    inf * 0 and inf + -inf are NaN; inf * x for x != 0 is an infinity of the
    product's sign)."""
    inf, nan = float("inf"), float("nan")
    # (acc, scale, bias, relu, expected)
    cases = [
        (0, inf, 0.0, False, 0), (0, -inf, 0.0, True, 0),          # inf * 0 = NaN
        (5, inf, 0.0, False, 127), (-5, inf, 0.0, False, -128),    # signed infinities
        (-5, inf, 0.0, True, 0), (5, -inf, 0.0, False, -128),
        (7, nan, 0.0, False, 0), (7, nan, 3.0, True, 0),           # NaN scale
        (3, 0.5, nan, False, 0), (-3, 0.5, nan, True, 0),          # NaN bias
        (3, 0.5, inf, False, 127), (3, 0.5, -inf, False, -128),   # infinite bias
        (3, 0.5, -inf, True, 0),
        (4, inf, -inf, False, 0), (-4, inf, inf, True, 0),         # inf - inf = NaN
        (100, 1e30, 1.0, False, 127), (-100, 1e30, 1.0, False, -128),  # overflow to inf
    ]
    acc = np.array([c[0] for c in cases], dtype=np.int64)
    sc = np.array([c[1] for c in cases], dtype=np.float32)
    bi = np.array([c[2] for c in cases], dtype=np.float32)
    ch = np.arange(acc.size, dtype=np.int64)
    for relu in (False, True):
        got = orc.requant_values(acc, ch, scale=sc, bias=bi, relu=relu)
        for i, (a, s_, b, r, want) in enumerate(cases):
            if r == relu:
                assert int(got[i]) == want, (a, s_, b, relu, int(got[i]), want)


def check_requant_conv(orc) -> None:
    """The fused entry = the INT32 convolution followed by the exact epilogue,
    with per-output-channel scale and bias, into a strided INT8 output."""
    rng = np.random.default_rng(31)
    x = rand_i8(rng, (2, 5, 7, 6))
    w = rand_i8(rng, (6, 5, 3, 2))
    a = dict(pre=(1, 0), post=(2, 1), stride=(2, 1), dil=(1, 2))
    y = orc.conv_fprop(x, w, **a).numpy().astype(np.int64)
    N, K, P, Q = y.shape
    sc = (rng.choice([-1, 1], K) * 2.0 ** rng.uniform(-9, -4, K)).astype(np.float32)
    bi = rng.uniform(-40, 40, K).astype(np.float32)
    for relu in (False, True):
        base = torch.full((N, P, Q, 2 * K), 99, dtype=torch.int8)
        out = base[..., ::2].permute(0, 3, 1, 2)         # NHWC view with gaps
        orc.conv_fprop_requant(x, w, scale=sc, bias=bi, relu=relu, out=out, **a)
        want = np.array([[[[exact_requant(y[n, k, p, q], sc[k], bi[k], relu) for q in range(Q)]
                           for p in range(P)] for k in range(K)] for n in range(N)], dtype=np.int8)
        assert np.array_equal(out.numpy(), want)
        assert (base[..., 1::2] == 99).all()
    # alpha with no arrays
    got = orc.conv_fprop_requant(x, w, alpha=0.125, **a).numpy()
    want = np.vectorize(lambda v: exact_requant(int(v), 0.125, 0.0, False))(y).astype(np.int8)
    assert np.array_equal(got, want)


def _scipy_true_conv(x: np.ndarray, w: np.ndarray, pre, post, stride, dil) -> np.ndarray:
    """Channel sums of scipy's 2-D convolution ('valid' after explicit zero
    padding; dilation by zero insertion between taps; stride by subsampling)."""
    from scipy.signal import convolve2d
    x = np.asarray(x, dtype=np.int64)
    w = np.asarray(w, dtype=np.int64)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    xp = np.pad(x, ((0, 0), (0, 0), (pre[0], post[0]), (pre[1], post[1])))
    wd = np.zeros((K, C, (R - 1) * dil[0] + 1, (S - 1) * dil[1] + 1), dtype=np.int64)
    wd[:, :, ::dil[0], ::dil[1]] = w
    out = None
    for n in range(N):
        rows = []
        for k in range(K):
            acc = sum(convolve2d(xp[n, c], wd[k, c], mode="valid") for c in range(C))
            rows.append(acc[::stride[0], ::stride[1]])
        out = np.stack(rows)[None] if out is None else np.concatenate([out, np.stack(rows)[None]])
    return out


def check_convolution_mode(orc) -> None:
    """Mode 1 = textbook convolution (scipy) and = brute-force
    cross-correlation with the filter reversed; mode 0 differs from it for
    asymmetric filters; a delta filter moves the image the other way."""
    rng = np.random.default_rng(37)
    for t in range(40):
        N, C, K = (int(v) for v in rng.integers(1, 4, 3))
        H, W = (int(v) for v in rng.integers(2, 9, 2))
        R, S = (int(v) for v in rng.integers(1, 4, 2))
        pre = tuple(int(v) for v in rng.integers(0, 3, 2))
        post = tuple(int(v) for v in rng.integers(0, 3, 2))
        st = tuple(int(v) for v in rng.integers(1, 3, 2))
        dl = tuple(int(v) for v in rng.integers(1, 3, 2))
        if H + pre[0] + post[0] - dl[0] * (R - 1) - 1 < 0 or W + pre[1] + post[1] - dl[1] * (S - 1) - 1 < 0:
            continue
        x = rand_i8(rng, (N, C, H, W))
        w = rand_i8(rng, (K, C, R, S))
        y1 = orc.conv_fprop(x, w, pre, post, st, dl, mode=1).numpy().astype(np.int64)
        assert np.array_equal(y1, _scipy_true_conv(x.numpy(), w.numpy(), pre, post, st, dl)), t
        wf = np.ascontiguousarray(w.numpy()[:, :, ::-1, ::-1])
        assert np.array_equal(y1, brute_force(x.numpy(), wf, pre, post, st, dl)), t
    # delta at (r0, s0) = (0, 2) of a 3x3 filter, no padding: cross-correlation
    # reads x[p + 0, q + 2], convolution x[p + 2, q + 0]
    x = rand_i8(rng, (1, 1, 6, 7))
    w = torch.zeros((1, 1, 3, 3), dtype=torch.int8)
    w[0, 0, 0, 2] = 1
    xn = x.numpy().astype(np.int64)[0, 0]
    assert np.array_equal(orc.conv_fprop(x, w).numpy()[0, 0], xn[0:4, 2:7])
    assert np.array_equal(orc.conv_fprop(x, w, mode=1).numpy()[0, 0], xn[2:6, 0:5])
    # the points and requantising entries take the mode too
    x = rand_i8(rng, (2, 3, 6, 5))
    w = rand_i8(rng, (4, 3, 3, 2))
    y1 = orc.conv_fprop(x, w, (1, 0), (0, 1), mode=1).numpy()
    idx = np.array([[n, k, p, q] for n in range(2) for k in range(4) for p in range(y1.shape[2])
                    for q in range(y1.shape[3])], dtype=np.int64)
    v = orc.conv_fprop_points(x, w, idx, (1, 0), (0, 1), mode=1)
    assert np.array_equal(v, y1[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]].astype(np.int64))
    q8 = orc.conv_fprop_requant(x, w, (1, 0), (0, 1), alpha=0.01, mode=1).numpy()
    want = np.vectorize(lambda a: exact_requant(int(a), 0.01, 0.0, False))(y1).astype(np.int8)
    assert np.array_equal(q8, want)


def autograd_dgrad(dy: torch.Tensor, w: torch.Tensor, xdims, pre, post, stride, dil) -> torch.Tensor:
    """d/dX of sum(conv2d(pad(X), W) * dY) in float64 (cross-correlation)."""
    x = torch.zeros(tuple(xdims), dtype=torch.float64, requires_grad=True)
    y = F.conv2d(F.pad(x, (pre[1], post[1], pre[0], post[0])), w.to(torch.float64),
                 stride=tuple(stride), dilation=tuple(dil))
    (g,) = torch.autograd.grad(y, x, dy.to(torch.float64))
    return g.round().to(torch.int64)


def check_dgrad(orc) -> None:
    """dgrad = float64 autograd of the forward (mode 0; mode 1 with the filter
    reversed), and the adjoint identity against the forward oracle, on random
    problems with padding, stride (up to 3) and dilation."""
    rng = np.random.default_rng(41)
    done = 0
    while done < 40:
        N, C, K = (int(v) for v in rng.integers(1, 4, 3))
        H, W = (int(v) for v in rng.integers(1, 10, 2))
        R, S = (int(v) for v in rng.integers(1, 4, 2))
        pre = tuple(int(v) for v in rng.integers(0, 3, 2))
        post = tuple(int(v) for v in rng.integers(0, 3, 2))
        st = tuple(int(v) for v in rng.integers(1, 4, 2))
        dl = tuple(int(v) for v in rng.integers(1, 3, 2))
        if H + pre[0] + post[0] - dl[0] * (R - 1) - 1 < 0 or W + pre[1] + post[1] - dl[1] * (S - 1) - 1 < 0:
            continue
        done += 1
        x = rand_i8(rng, (N, C, H, W))
        w = rand_i8(rng, (K, C, R, S))
        yd = orc.out_dims(x.shape, w.shape, pre, post, st, dl)
        dy = rand_i8(rng, yd)
        for mode in (0, 1):
            dx = orc.conv_dgrad(dy, w, x.shape, pre, post, st, dl, mode=mode).to(torch.int64)
            wm = w if mode == 0 else w.flip(2, 3).contiguous()
            assert torch.equal(dx, autograd_dgrad(dy, wm, x.shape, pre, post, st, dl)), (done, mode)
            y = orc.conv_fprop(x, w, pre, post, st, dl, mode=mode).to(torch.int64)
            assert int((y * dy.to(torch.int64)).sum()) == int((x.to(torch.int64) * dx).sum())
    # strided output and a dy view with gaps
    x = rand_i8(rng, (2, 3, 7, 6))
    w = rand_i8(rng, (4, 3, 3, 3))
    yd = orc.out_dims(x.shape, w.shape, (1, 1), (1, 1), (2, 2), (1, 1))
    big = rand_i8(rng, (yd[0], yd[1], yd[2], 2 * yd[3]))
    dy = big[..., ::2]
    base = torch.full((2, 7, 6, 2 * 3), 5, dtype=torch.int32)
    out = base[..., ::2].permute(0, 3, 1, 2)
    orc.conv_dgrad(dy, w, None, (1, 1), (1, 1), (2, 2), (1, 1), out=out)
    assert torch.equal(out.to(torch.int64),
                       autograd_dgrad(dy.contiguous(), w, x.shape, (1, 1), (1, 1), (2, 2), (1, 1)))
    assert (base[..., 1::2] == 5).all()


def autograd_wgrad(x: torch.Tensor, dy: torch.Tensor, wdims, pre, post, stride, dil) -> torch.Tensor:
    """d/dW of sum(conv2d(pad(X), W) * dY) in float64 (cross-correlation)."""
    w = torch.zeros(tuple(wdims), dtype=torch.float64, requires_grad=True)
    y = F.conv2d(F.pad(x.to(torch.float64), (pre[1], post[1], pre[0], post[0])), w,
                 stride=tuple(stride), dilation=tuple(dil))
    (g,) = torch.autograd.grad(y, w, dy.to(torch.float64))
    return g.round().to(torch.int64)


def check_wgrad(orc) -> None:
    """wgrad = float64 autograd of the forward with respect to the filter
    (mode 1: reversed taps), and <fprop(X, W), dY> = <W, wgrad(X, dY)>."""
    rng = np.random.default_rng(47)
    done = 0
    while done < 40:
        N, C, K = (int(v) for v in rng.integers(1, 4, 3))
        H, W = (int(v) for v in rng.integers(1, 10, 2))
        R, S = (int(v) for v in rng.integers(1, 4, 2))
        pre = tuple(int(v) for v in rng.integers(0, 3, 2))
        post = tuple(int(v) for v in rng.integers(0, 3, 2))
        st = tuple(int(v) for v in rng.integers(1, 4, 2))
        dl = tuple(int(v) for v in rng.integers(1, 3, 2))
        if H + pre[0] + post[0] - dl[0] * (R - 1) - 1 < 0 or W + pre[1] + post[1] - dl[1] * (S - 1) - 1 < 0:
            continue
        done += 1
        x = rand_i8(rng, (N, C, H, W))
        w = rand_i8(rng, (K, C, R, S))
        dy = rand_i8(rng, orc.out_dims(x.shape, w.shape, pre, post, st, dl))
        for mode in (0, 1):
            dw = orc.conv_wgrad(x, dy, w.shape, pre, post, st, dl, mode=mode).to(torch.int64)
            ref = autograd_wgrad(x, dy, w.shape, pre, post, st, dl)
            if mode:
                ref = ref.flip(2, 3)
            assert torch.equal(dw, ref), (done, mode)
            y = orc.conv_fprop(x, w, pre, post, st, dl, mode=mode).to(torch.int64)
            assert int((y * dy.to(torch.int64)).sum()) == int((w.to(torch.int64) * dw).sum())
    # strided views in and out
    x = rand_i8(rng, (3, 4, 8, 7))
    dy_full = rand_i8(rng, (3, 5, 8, 2 * 7))
    dy = dy_full[..., ::2]                           # 3x5x8x7: 3x3 filter, pad 1, stride 1
    base = torch.full((4, 5, 3, 3), 9, dtype=torch.int32)
    out = base.permute(1, 0, 2, 3)                   # [K, C, R, S] view of a [C, K, R, S] buffer
    orc.conv_wgrad(x, dy, None, 1, 1, 1, 1, out=out)
    assert torch.equal(out.to(torch.int64), autograd_wgrad(x, dy.contiguous(), (5, 4, 3, 3), (1, 1),
                                                          (1, 1), (1, 1), (1, 1)))


QUICK_CHECKS = [
    check_random_vs_brute_force, check_offcentre_delta, check_identity_1x1, check_ones_count,
    check_constant_min, check_layouts, check_metamorphic, check_points, check_requant_exact,
    check_requant_nonfinite, check_requant_conv, check_convolution_mode, check_dgrad, check_wgrad,
]
