"""Per-workgroup phase timeline of the 3x3 ring kernel (instrumented build).

The library built with CONV_I8_PHASE_CLOCK has the 3x3 ring kernel stamp the
shader clock (s_memtime) at the ends of its phases and write the stamps, with
the constant 100 MHz clock at its start and end, to a device buffer set by
conv_i8_set_phase_clock.  Nothing else changes: the stamps add a few scalar
instructions per workgroup.  This module builds that library next to the
product one (`--build`, on any host with hipcc) and, on a GPU, times the
instrumented call on a workload and reports where a workgroup spends its time:

- arguments: kernel entry to the argument block loaded,
- prologue: to the first MFMA fragments read (the loads of block 0),
- main loop: the channel blocks before the last one,
- tail: the last block, row block by row block, with its stores,
- in-workgroup total, and what the call takes beyond it (launch, dispatch,
  the end-of-kernel write-back) from HIP events around the timed calls.

The product library and the instrumented one with its stamps switched off
are timed first, so the output states what the instrumentation costs.

    python -m int8_convolution_forward_amd.phase_clock --build
    python -m int8_convolution_forward_amd.phase_clock [--workloads a,b] [--calls N]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import subprocess
import sys

from . import build as _build

LIB = os.path.join(_build.LIB_DIR, "libconv_i8_phases.so")
SLOTS = 16


def build_instrumented(verbose: bool = False) -> str:
    os.makedirs(_build.LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [_build.HIPCC, *_build.HIP_FLAGS, "-DCONV_I8_PHASE_CLOCK", "-I", _build.INCLUDE, "-I", _build.CSRC,
           *_build.SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def timeline(name: str, calls: int = 300, warmup: int = 1000, log=sys.stdout) -> dict:
    """Phase means (µs) over the workgroups of the last of `calls` timed calls
    of conv_fprop_i8_ws on workload `name`, rotating buffer sets."""
    import torch

    import int8_convolution_forward_amd as ci8
    import workloads as wl

    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB}: run with --build first")
    lib = ctypes.CDLL(LIB)
    lib.conv_fprop_i8_ws.argtypes = ci8.lib.conv_fprop_i8_ws.argtypes
    lib.conv_fprop_i8_ws.restype = ctypes.c_int
    lib.conv_i8_set_phase_clock.argtypes = [ctypes.c_void_p]
    lib.conv_i8_set_phase_clock.restype = ctypes.c_int
    c = wl.case(name)
    dev = torch.device("cuda:0")
    d = wl.make_inputs(c, c.seed_base)
    plan = ci8.plan_fields(ci8.conv_fprop_i8_plan(ci8.desc(c.image.dims, c.image.strides, ci8.DT_INT8),
                                                  ci8.desc(c.filter.dims, c.filter.strides, ci8.DT_INT8),
                                                  ci8.desc(c.out.dims, c.out.strides, ci8.DT_INT32),
                                                  c.pre, c.post, c.stride, c.dilation))
    if not plan["tile"].startswith("t"):
        raise ValueError(f"{name}: planned on {plan['tile']}, not a 3x3 ring tail tile")
    sets = []
    for _ in range(8):
        x = wl.to_device(d["x_storage"], c.image, dev)
        w = wl.to_device(d["w_storage"], c.filter, dev)
        y = torch.empty(c.out.storage_size, dtype=torch.int32, device=dev)
        sets.append((x, w, y, torch.as_strided(y, c.out.dims, c.out.strides, c.out.offset)))
    tiles = int(plan["tiles"])
    # room for more workgroups than the plan says (the buffer outlives no call)
    stamps = torch.zeros(SLOTS * max(tiles, 4096), dtype=torch.int64, device=dev)
    params = ci8._params(c.pre, c.post, c.stride, c.dilation, None)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [(ctypes.byref(ci8.desc(s[0][1])), ctypes.c_void_p(s[0][1].data_ptr()),
             ctypes.byref(ci8.desc(s[1][1])), ctypes.c_void_p(s[1][1].data_ptr()),
             ctypes.byref(ci8.desc(s[3])), ctypes.c_void_p(s[3].data_ptr()), *params, None, ctypes.c_size_t(0), sh)
            for s in sets]

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    def call(lib_):
        def fn(i):
            rc = lib_.conv_fprop_i8_ws(*args[i % len(args)])
            if rc:
                raise RuntimeError(ci8.status_string(rc))
        return fn

    # the product library, then the instrumented one without and with stamps:
    # the difference is what the instrumentation costs
    us_product = timed(call(ci8.lib))
    lib.conv_i8_set_phase_clock(None)
    us_off = timed(call(lib))
    lib.conv_i8_set_phase_clock(ctypes.c_void_p(stamps.data_ptr()))
    us_call = timed(call(lib))
    lib.conv_i8_set_phase_clock(None)
    t = stamps[:SLOTS * tiles].view(tiles, SLOTS).cpu().double()
    ghz = float(((t[:, 11] - t[:, 0]) / ((t[:, 15] - t[:, 14]) / 100e6)).mean()) / 1e9

    def span(a, b):
        return float(((t[:, b] - t[:, a]) / (ghz * 1e3)).mean())

    res = {"workload": name, "tile": plan["tile"], "workgroups": tiles, "us_per_call_product": us_product,
           "us_per_call_stamps_off": us_off, "us_per_call": us_call, "shader_ghz": ghz,
           "arguments": span(0, 1), "prologue": span(0, 4), "main_loop": span(4, 5),
           "tail": span(5, 11), "in_workgroup": span(0, 11),
           "start_spread_us": float((t[:, 14].max() - t[:, 14].min()) / 100.0)}
    res["outside_workgroup"] = us_call - res["in_workgroup"]
    print(f"{name} ({plan['tile']}, {tiles} workgroups): per call {us_product:.2f} us (product library), "
          f"{us_off:.2f} (instrumented, stamps off), {us_call:.2f} (stamps on: the run below); shader clock "
          f"{ghz:.3f} GHz; per workgroup: arguments {res['arguments']:.2f}, prologue {res['prologue']:.2f}, "
          f"main loop {res['main_loop']:.2f}, tail {res['tail']:.2f}, in-workgroup {res['in_workgroup']:.2f}; "
          f"outside the workgroups {res['outside_workgroup']:.2f}; start spread {res['start_spread_us']:.2f} us",
          file=log, flush=True)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--build", action="store_true", help="build the instrumented library and exit")
    ap.add_argument("--workloads", default="large_channel_n64_c512_14,bottleneck_3x3_n32_c128_28")
    ap.add_argument("--calls", type=int, default=300)
    args = ap.parse_args(argv)
    if args.build:
        print(build_instrumented(verbose=True))
        return
    for n in args.workloads.split(","):
        timeline(n, calls=args.calls)


if __name__ == "__main__":
    main()
