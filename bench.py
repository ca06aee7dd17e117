"""Benchmark: INT8 conv_fprop throughput on one MI355X.

One step = one conv_fprop_i8 call (the whole path: layout normalisation if
the operands need it, implicit-GEMM kernel with its epilogue) over one batch
of seeded synthetic input that is already resident in HBM.  With
``--epilogue requant`` a step is one conv_fprop_i8_requant call instead (INT8
output through the fused scale / bias / ReLU / saturation epilogue).  Inputs and
outputs rotate over enough buffer sets (> 512 MB) that the 256 MB Infinity
Cache cannot serve a step from a previous one.

Prints one JSON line: the metric (TOPS = 2*N*K*P*Q*C*R*S / s), ms per step,
the roofline of the implicit-GEMM kernel timed alone with HIP events on the
launch stream, and the CPU oracle timed on the host as a baseline.  Each GPU
figure is the median of five timed batches of ``--steps`` steps (every batch
between two device synchronisations, its events on the launch stream); the
five batch times are reported beside it.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT8 conv_fprop TOPS (2·NKPQ·CRS/s) and % of MI355X INT8 MFMA peak"
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
DEFAULT_WORKLOAD = "large_channel_n64_c512_14"
TIMED_BATCHES = 5
# kernel names as the profiler lists them, by plan tile
RING9_TILES = ("r256x128", "t256x128", "t128x128")


def timed_batches(run, stream, steps):
    """ms per step of TIMED_BATCHES batches, each of `steps` steps run by
    run(), timed with events on the launch stream between device
    synchronisations."""
    import torch

    out = []
    for _ in range(TIMED_BATCHES):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def mfma_ceiling(ci8, stream, workgroup_counts, iters=2048, launches=10):
    """TOP/s of the matrix-core calibration kernel (random INT8 operands in
    registers, back-to-back v_mfma_i32_32x32x32_i8, one workgroup of four
    waves per CU) on each workgroup count: median of five timed batches."""
    import torch

    out = torch.empty(max(workgroup_counts) * 256, dtype=torch.int32, device="cuda")
    seed = 0x9E3779B9
    res = {}
    for wg in workgroup_counts:
        def run():
            for _ in range(launches):
                ci8.conv_i8_mfma_ceiling(wg, iters, seed, out, stream)

        run()
        torch.cuda.synchronize()
        ms = median(timed_batches(run, stream, launches))
        res[str(wg)] = wg * 4 * iters * 8 * 65536 / (ms * 1e-3) / 1e12
    return res


def launch_floor(ci8, workgroups, launches=200):
    """Device µs per launch of a kernel that does almost nothing (the
    calibration kernel with zero operands and one iteration: eight MFMAs and
    a 128-value sum per wave) on `workgroups` workgroups, `launches` of them
    recorded in one HIP graph so that the host's launch rate does not enter:
    the floor under every launch (dispatch, kernel end, the end-of-kernel
    write-back), median of five replays."""
    import torch

    out = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ci8.conv_i8_mfma_ceiling(workgroups, 1, 0, out, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for _ in range(launches):
            ci8.conv_i8_mfma_ceiling(workgroups, 1, 0, out, cap)
    g.replay()
    torch.cuda.synchronize()
    return median(timed_batches(g.replay, torch.cuda.current_stream(), launches)) * 1e3


def host_description(orc):
    """nproc, the CPU model and the oracle's thread count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "oracle_threads": orc.max_threads()}


def single_core_small_configs(orc):
    """The oracle on one thread over the two smallest workloads (the tiny
    5x5 and the stride-2 downsample layer), whole problem once each."""
    import workloads as wl

    res = {}
    for name in ("tiny_5x5_r3", "downsample_s2_n8_c64_56"):
        c = wl.case(name)
        d = wl.make_inputs(c, c.seed_base)
        t0 = time.perf_counter()
        orc.conv_fprop(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation, threads=1)
        el = time.perf_counter() - t0
        res[name] = {"seconds": el, "GOPS": c.ops / el / 1e9}
    return res


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first; the GPU needs some tens of ms of load to settle its clock")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--graph", action="store_true",
                    help="record the timed steps into one HIP graph (captured through the "
                         "workspace entry) and time its replay")
    ap.add_argument("--mode", choices=("cross_correlation", "convolution"),
                    default="cross_correlation",
                    help="convolution: true convolution (filter taps reversed) through the "
                         "general entry conv_fprop_i8_ex_ws")
    ap.add_argument("--op", choices=("fprop", "dgrad", "wgrad"), default="fprop",
                    help="dgrad: the data gradient of the workload (loss shaped like its output, "
                         "INT32 result shaped like its image) through conv_dgrad_i8_ws; wgrad: "
                         "the weight gradient (the workload's image and such a loss, INT32 "
                         "result shaped like its filter) through conv_wgrad_i8_ws")
    ap.add_argument("--epilogue", choices=("int32", "requant"), default="int32",
                    help="int32: the plain entry; requant: INT8 output with per-channel "
                         "scale and bias and ReLU")
    ap.add_argument("--rotate-mb", type=float, default=600.0)
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    return ap.parse_args()


def input_seed(args, c) -> int:
    """Seed of the timed inputs: --seed, else the workload's own."""
    return c.seed_base if args.seed is None else args.seed


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int8_convolution_forward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, launch_bytes_alg: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def bench_grad(args, c):
    """Whole-call timing of a gradient.  dgrad: dY (INT8, the forward output's
    dims and strides), the workload's filter, dX (INT32, the image dims,
    channels_last); every call repacks the transposed filter and runs one
    forward convolution per stride phase.  wgrad: the workload's image, such a
    dY, dW (INT32, the filter's dims and strides); one forward convolution of
    the transposed operands (both repacked)."""
    import torch

    import int8_convolution_forward_amd as ci8
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.make_inputs(c, input_seed(args, c))
    N, K, P, Q = c.out.dims
    _, C, R, S = c.filter.dims
    H, W = c.image.dims[2], c.image.dims[3]
    ops = c.ops
    mode = 1 if args.mode == "convolution" else 0
    g = torch.Generator().manual_seed(input_seed(args, c) + 91)
    dy0 = torch.randint(-128, 128, (c.out.storage_size,), dtype=torch.int8, generator=g).to(dev)
    wg = args.op == "wgrad"
    if wg:
        w0, _ = wl.to_device(d["x_storage"], c.image, dev)     # the image
        in_spec = c.image
        res_dims, res_strides = c.filter.dims, c.filter.strides
    else:
        w0, _ = wl.to_device(d["w_storage"], c.filter, dev)
        in_spec = c.filter
        res_dims, res_strides = c.image.dims, wl.channels_last_strides(c.image.dims)
    dx_strides = res_strides
    dx_size = wl.TensorSpec(res_dims, res_strides).storage_size
    set_bytes = dy0.numel() + w0.numel() + 4 * dx_size
    nsets = max(2, min(128, int(args.rotate_mb * 2**20 // set_bytes) + 1))
    sets = []
    for _ in range(nsets):
        dys, ws_ = dy0.clone(), w0.clone()
        dxs = torch.empty(dx_size, dtype=torch.int32, device=dev)
        dyv = torch.as_strided(dys, c.out.dims, c.out.strides)
        inv = torch.as_strided(ws_, in_spec.dims, in_spec.strides, in_spec.offset)
        resv = torch.as_strided(dxs, res_dims, res_strides)
        # argument order of the C entry: dgrad (loss, filter, dx), wgrad (image, loss, dw)
        sets.append((dys, ws_, dxs, inv, dyv, resv) if wg else (dys, ws_, dxs, dyv, inv, resv))
    wsize = ci8.conv_wgrad_i8_workspace_size if wg else ci8.conv_dgrad_i8_workspace_size
    ws_bytes = wsize(sets[0][3], sets[0][4], sets[0][5], c.pre, c.post, c.stride, c.dilation,
                     mode=mode)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    params = ci8._params(c.pre, c.post, c.stride, c.dilation, None)
    calls = [(ctypes.byref(ci8.desc(s_[3])), ctypes.c_void_p(s_[3].data_ptr()),
              ctypes.byref(ci8.desc(s_[4])), ctypes.c_void_p(s_[4].data_ptr()),
              ctypes.byref(ci8.desc(s_[5])), ctypes.c_void_p(s_[5].data_ptr()), *params,
              ctypes.c_int32(mode), ctypes.c_void_p(workspace.data_ptr()) if ws_bytes else None,
              ctypes.c_size_t(ws_bytes), sh) for s_ in sets]
    fn = ci8.lib.conv_wgrad_i8_ws if wg else ci8.lib.conv_dgrad_i8_ws

    def step(i):
        rc = fn(*calls[i % nsets])
        if rc != 0:
            raise RuntimeError(ci8.status_string(rc))

    print(f"bench: {args.op} of {c.name}; {nsets} buffer sets of {set_bytes / 2**20:.1f} MiB, "
          f"workspace {ws_bytes} B", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def run():
        for i in range(args.steps):
            step(i)

    batches = timed_batches(run, stream, args.steps)
    ms = median(batches)
    tops = ops / (ms * 1e-3) / 1e12
    alg_bytes = (N * K * P * Q + N * C * H * W + 4 * K * C * R * S) if wg else \
        (N * K * P * Q + K * C * R * S + 4 * N * C * H * W)
    ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ops / alg_bytes >= ridge:
        roof = {"bound": "mfma", "achieved": tops, "peak": INT8_PEAK_TOPS, "unit": "TOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    plan = ci8.conv_wgrad_i8_plan(sets[0][3], sets[0][4], sets[0][5], c.pre, c.post, c.stride, c.dilation,
                                  mode=mode) if wg else None
    if wg and ci8.plan_fields(plan).get("kernel") == "wgrad_in_place":
        what = "whole wgrad call (the in-place kernel reading both operands + the sum of its partial copies)"
    elif wg:
        what = "whole wgrad call (repacks of both transposed operands + one forward kernel)"
    else:
        what = "whole dgrad call (filter repack + one forward kernel per stride phase)"
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": None,
                 "kernel": what,
                 "kernel_avg_us": ms * 1e3, "kernel_only_launch": False,
                 "timed_batches_ms_per_step": batches,
                 "algorithmic_bytes": alg_bytes, "algorithmic_ops": ops})
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.load()
        threads = orc.max_threads()
        dy_cpu = torch.as_strided(dy0.cpu(), c.out.dims, c.out.strides)
        tt = time.perf_counter()
        reps = 0
        while True:
            if wg:
                orc.conv_wgrad(d["x"], dy_cpu, c.filter.dims, c.pre, c.post, c.stride, c.dilation,
                               threads=threads, mode=mode)
            else:
                orc.conv_dgrad(dy_cpu, d["w"], c.image.dims, c.pre, c.post, c.stride, c.dilation,
                               threads=threads, mode=mode)
            reps += 1
            el = time.perf_counter() - tt
            if el >= args.cpu_seconds or reps >= 20:
                break
        cpu = {"value": ops * reps / el / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
               "sample": f"the whole {args.op} of {c.name}, {reps} run(s), {el:.1f} s wall, "
                         f"{threads} OpenMP threads",
               "host": host_description(orc)}
    out = {
        "metric": METRIC, "value": tops, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "timed_batches_ms_per_step": batches,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": c.name, "seed": input_seed(args, c), "op": args.op, "mode": args.mode,
                   "loss": list(c.out.dims), "loss_strides": list(c.out.strides),
                   ("image" if wg else "filter"): list(in_spec.dims),
                   ("image_strides" if wg else "filter_strides"): list(in_spec.strides),
                   ("dw" if wg else "dx"): list(res_dims),
                   ("dw_strides" if wg else "dx_strides"): list(dx_strides),
                   "pre_padding": list(c.pre), "post_padding": list(c.post),
                   "stride": list(c.stride), "dilation": list(c.dilation),
                   "accumulate": "int32", "output": "int32", "buffer_sets": nsets,
                   **({"plan": plan} if plan else {})},
        "frac_of_int8_peak": tops / INT8_PEAK_TOPS,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the convolution shards over the "
              "batch with no exchange, but no multi-GPU run is provided (--gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import int8_convolution_forward_amd as ci8
    import workloads as wl

    c = wl.case(args.workload)
    if args.op in ("dgrad", "wgrad"):
        return bench_grad(args, c)
    rq_on = args.epilogue == "requant"
    esize = 1 if rq_on else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = wl.make_inputs(c, input_seed(args, c))
    N, K, P, Q = c.out.dims
    _, C, R, S = c.filter.dims
    ops = c.ops

    # ---- resident, rotating buffer sets --------------------------------
    x0_storage, _ = wl.to_device(d["x_storage"], c.image, dev)
    w0_storage, _ = wl.to_device(d["w_storage"], c.filter, dev)
    set_bytes = (x0_storage.numel() + w0_storage.numel() + esize * c.out.storage_size)
    nsets = max(2, min(128, int(args.rotate_mb * 2**20 // set_bytes) + 1))
    sets = []
    for i in range(nsets):
        xs = x0_storage.clone()
        ws_ = w0_storage.clone()
        ys = torch.empty(c.out.storage_size, dtype=torch.int8 if rq_on else torch.int32, device=dev)
        x = torch.as_strided(xs, c.image.dims, c.image.strides, c.image.offset)
        w = torch.as_strided(ws_, c.filter.dims, c.filter.strides, c.filter.offset)
        y = torch.as_strided(ys, c.out.dims, c.out.strides, c.out.offset)
        sets.append((xs, ws_, ys, x, w, y))
    # requantisation parameters: per-channel scales that keep typical sums of
    # random operands around +-64, biases, ReLU (all on the device)
    g = torch.Generator().manual_seed(input_seed(args, c) + 77)
    typical = (C * R * S) ** 0.5 * 128 * 128 / 3
    q_scale = ((torch.rand(K, generator=g) + 0.5) * 64 / typical).to(dev)
    q_bias = ((torch.rand(K, generator=g) - 0.5) * 40).to(dev)
    rq = ci8.Requant(q_scale.data_ptr(), 1.0, q_bias.data_ptr(), 1)
    # the plan depends on the output strides, not on its dtype
    out32 = ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT32)
    wsize = ci8.conv_fprop_i8_requant_workspace_size if rq_on else ci8.conv_fprop_i8_workspace_size
    ws_bytes = wsize(sets[0][3], sets[0][4], sets[0][5], c.pre, c.post, c.stride, c.dilation)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    plan = ci8.conv_fprop_i8_plan(sets[0][3], sets[0][4], out32, c.pre, c.post, c.stride,
                                  c.dilation)

    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    params = ci8._params(c.pre, c.post, c.stride, c.dilation, None)

    conv_mode = 1 if args.mode == "convolution" else 0

    def prebuilt(x, w, y):
        if conv_mode:
            extra = (ctypes.c_int32(conv_mode), ctypes.byref(rq) if rq_on else None)
        else:
            extra = (ctypes.byref(rq),) if rq_on else ()
        return (ctypes.byref(ci8.desc(x)), ctypes.c_void_p(x.data_ptr()),
                ctypes.byref(ci8.desc(w)), ctypes.c_void_p(w.data_ptr()),
                ctypes.byref(ci8.desc(y)), ctypes.c_void_p(y.data_ptr()), *params, *extra,
                ctypes.c_void_p(workspace.data_ptr()) if ws_bytes else None,
                ctypes.c_size_t(ws_bytes), sh)

    calls = [prebuilt(s[3], s[4], s[5]) for s in sets]
    if conv_mode:
        fn = ci8.lib.conv_fprop_i8_ex_ws
    else:
        fn = ci8.lib.conv_fprop_i8_requant_ws if rq_on else ci8.lib.conv_fprop_i8_ws

    def step(i):
        rc = fn(*calls[i % nsets])
        if rc != 0:
            raise RuntimeError(ci8.status_string(rc))

    print(f"bench: {c.name} plan: {plan}; {nsets} buffer sets of {set_bytes / 2**20:.1f} MiB",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps per batch ------------------
    if args.graph:
        # the same calls, recorded on the capture stream, replayed as one graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            gcalls = [c_[:-1] + (ctypes.c_void_p(cap.cuda_stream),) for c_ in calls]
            for i in range(args.steps):
                rc = fn(*gcalls[i % nsets])
                if rc != 0:
                    raise RuntimeError(ci8.status_string(rc))
        graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()

    def run():
        if args.graph:
            graph.replay()
        else:
            for i in range(args.steps):
                step(i)

    batches = timed_batches(run, stream, args.steps)
    ms_per_step = median(batches)
    tops = ops / (ms_per_step * 1e-3) / 1e12
    print(f"bench: {ms_per_step * 1e3:.2f} us/step, {tops:.1f} TOPS", file=sys.stderr, flush=True)

    # ---- implicit-GEMM kernel alone: back-to-back launches between two
    # events on the launch stream, average duration per launch ------------
    # Operands that the whole path would repack are given to it already
    # channel-innermost, so each call is exactly one implicit-GEMM launch.
    kcalls = []
    for s in sets:
        x, w, y = s[3], s[4], s[5]
        f = ci8.plan_fields(ci8.conv_fprop_i8_plan(x, w, out32, c.pre, c.post, c.stride, c.dilation))
        if f["repack_image"] == "1":
            x = x.contiguous(memory_format=torch.channels_last)
        if f["repack_filter"] == "1":
            w = w.contiguous(memory_format=torch.channels_last)
        kcalls.append((x, w, y))
    kf = ci8.plan_fields(ci8.conv_fprop_i8_plan(kcalls[0][0], kcalls[0][1], out32, c.pre, c.post,
                                                c.stride, c.dilation))
    kernel_only = kf["repack_image"] == "0" and kf["repack_filter"] == "0" and \
        wsize(*kcalls[0], c.pre, c.post, c.stride, c.dilation) == 0
    kpre = [prebuilt(*t) for t in kcalls]
    nk = max(args.steps, 50)
    for i in range(min(10, nk)):
        fn(*kpre[i % nsets])
    torch.cuda.synchronize()

    def krun():
        for i in range(nk):
            rc = fn(*kpre[i % nsets])
            if rc:
                raise RuntimeError(ci8.status_string(rc))

    kbatches = timed_batches(krun, stream, nk)
    k_avg_ms = median(kbatches)

    # algorithmic bytes: image, filter read once, output written once (int32,
    # or int8 plus the per-channel scale and bias)
    alg_bytes = N * C * c.image.dims[2] * c.image.dims[3] + K * C * R * S + esize * N * K * P * Q
    if rq_on:
        alg_bytes += 8 * K
    ai = ops / alg_bytes
    ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": ops / (k_avg_ms * 1e-3) / 1e12, "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (k_avg_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "mfma":
        # the measured ceiling beside the published peak: the rate the matrix
        # cores reach with random operands on as many CUs as the kernel's
        # grid covers, and on all 256 (the clock falls under the power limit)
        wgs = min(int(kf.get("tiles", "256")), 256)
        ceil = mfma_ceiling(ci8, stream, sorted({wgs, 256}))
        roof["mfma_ceiling"] = {"unit": "TOP/s", "operands": "random int8 in registers",
                                "tops_by_busy_cus": ceil}
        roof["frac_of_ceiling"] = roof["achieved"] / ceil[str(wgs)]
    floor_wgs = max(1, min(int(kf.get("tiles", "256")), 1 << 20))
    roof["launch_floor_us"] = {"workgroups": floor_wgs, "us": launch_floor(ci8, floor_wgs),
                               "launch": "hip graph of back-to-back near-empty kernels"}
    roof["traffic"] = traffic_from_profiles(c.name + ("_requant" if rq_on else ""), alg_bytes)
    if kf.get("tile") in RING9_TILES:
        roof["kernel"] = "conv_fp3x3_ring9_kernel"
    elif kf.get("kernel") == "footprint":
        roof["kernel"] = "conv_footprint3x3_kernel"
    elif kf.get("kernel") == "pointwise":
        roof["kernel"] = "conv_pointwise_kernel"
    elif kf.get("kernel") == "direct":
        roof["kernel"] = "conv_direct_kernel"
    else:
        roof["kernel"] = "conv_igemm_kernel"
    roof["kernel_tile"] = kf.get("tile")
    roof["kernel_avg_us"] = k_avg_ms * 1e3
    roof["kernel_timed_batches_us"] = [v * 1e3 for v in kbatches]
    roof["kernel_launches_timed"] = nk
    roof["kernel_only_launch"] = kernel_only
    roof["algorithmic_bytes"] = alg_bytes
    roof["algorithmic_ops"] = ops

    # ---- CPU oracle baseline (rank 0, one GPU) -------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.load()
        threads = orc.max_threads()
        t0 = time.perf_counter()
        reps = 0
        sc_cpu, bi_cpu = q_scale.cpu().numpy(), q_bias.cpu().numpy()
        while True:
            if rq_on:
                orc.conv_fprop_requant(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation,
                                       scale=sc_cpu, bias=bi_cpu, relu=True, threads=threads,
                                       mode=conv_mode)
            else:
                orc.conv_fprop(d["x"], d["w"], c.pre, c.post, c.stride, c.dilation, threads=threads,
                               mode=conv_mode)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps >= 20:
                break
        cpu = {"value": ops * reps / el / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
               "sample": f"the whole {c.name} workload, {reps} run(s), {el:.1f} s wall, "
                         f"{threads} OpenMP threads, plain -O2 C with int64 sums",
               "host": host_description(orc),
               "single_core": single_core_small_configs(orc)}

    out = {
        "metric": METRIC,
        "value": tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "timed_batches_ms_per_step": batches,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": c.name, "seed": input_seed(args, c), "image": list(c.image.dims), "image_strides": list(c.image.strides),
                   "filter": list(c.filter.dims), "filter_strides": list(c.filter.strides),
                   "out": list(c.out.dims), "out_strides": list(c.out.strides),
                   "pre_padding": list(c.pre), "post_padding": list(c.post),
                   "stride": list(c.stride), "dilation": list(c.dilation),
                   "accumulate": "int32",
                   "output": ("int8: fma(sum, per-channel scale, bias), ReLU, round half to "
                              "even, saturate") if rq_on else "int32",
                   "plan": plan, "launch": "hip graph replay" if args.graph else "eager",
                   "mode": args.mode,
                   "buffer_sets": nsets},
        "frac_of_int8_peak": tops / INT8_PEAK_TOPS,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
