"""Tile sweep: time every tile shape that applies to a problem, keep the fastest.

The cuDNN frontend tutorial page (its autotuning paragraph) builds every plan
the heuristics offer, times each one and ships the index of the fastest.  This
module does the same over the library's tile shapes (conv_i8_tile_names): for
each workload it forces each tile through CONV_I8_TILE, keeps the tiles the
planner accepts for that problem, times the whole conv_fprop_i8_ws call
(median of five batches over rotating HBM-resident buffer sets, so the
Infinity Cache cannot serve one call from the previous one) and reports the
table.  With --write it rewrites csrc/tuned_tiles.inc, the table the planner
consults before its cost model (rebuild the library afterwards).

    python -m int8_convolution_forward_amd.tune [--workloads a,b] [--write]

Run it from the repository root on the GPU the table is for.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys
import time

INC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tuned_tiles.inc")
BATCHES = 5


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def sweep(name, calls_per_batch=200, warmup=300, rotate_mb=600.0, log=sys.stderr):
    """[(tile, us)] for every tile the planner accepts on workload `name`,
    fastest first, plus the problem's table key."""
    import torch

    import int8_convolution_forward_amd as ci8
    import workloads as wl

    c = wl.case(name)
    dev = torch.device("cuda:0")
    d = wl.make_inputs(c, c.seed_base)
    x0, _ = wl.to_device(d["x_storage"], c.image, dev)
    w0, _ = wl.to_device(d["w_storage"], c.filter, dev)
    set_bytes = x0.numel() + w0.numel() + 4 * c.out.storage_size
    nsets = max(2, min(128, int(rotate_mb * 2**20 // set_bytes) + 1))
    sets = []
    for _ in range(nsets):
        xs, ws_ = x0.clone(), w0.clone()
        ys = torch.empty(c.out.storage_size, dtype=torch.int32, device=dev)
        sets.append((xs, ws_, ys, torch.as_strided(xs, c.image.dims, c.image.strides, c.image.offset),
                     torch.as_strided(ws_, c.filter.dims, c.filter.strides, c.filter.offset),
                     torch.as_strided(ys, c.out.dims, c.out.strides, c.out.offset)))
    params = ci8._params(c.pre, c.post, c.stride, c.dilation, None)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    saved = os.environ.pop("CONV_I8_TILE", None)
    results = []
    lanes = None
    try:
        for tile in ci8.conv_i8_tile_names():
            os.environ["CONV_I8_TILE"] = tile
            f = ci8.plan_fields(ci8.conv_fprop_i8_plan(sets[0][3], sets[0][4], sets[0][5], c.pre, c.post,
                                                       c.stride, c.dilation))
            lanes = f.get("lanes")
            if f.get("tile") != tile:
                continue        # does not apply to this problem
            wsb = ci8.conv_fprop_i8_workspace_size(sets[0][3], sets[0][4], sets[0][5], c.pre, c.post,
                                                   c.stride, c.dilation)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            calls = [(ctypes.byref(ci8.desc(s[3])), ctypes.c_void_p(s[3].data_ptr()),
                      ctypes.byref(ci8.desc(s[4])), ctypes.c_void_p(s[4].data_ptr()),
                      ctypes.byref(ci8.desc(s[5])), ctypes.c_void_p(s[5].data_ptr()), *params,
                      ctypes.c_void_p(ws.data_ptr()) if wsb else None, ctypes.c_size_t(wsb), sh)
                     for s in sets]
            fn = ci8.lib.conv_fprop_i8_ws

            def run(n):
                for i in range(n):
                    rc = fn(*calls[i % nsets])
                    if rc:
                        raise RuntimeError(ci8.status_string(rc))

            run(warmup)
            torch.cuda.synchronize()
            times = []
            for _ in range(BATCHES):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(calls_per_batch)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3 / calls_per_batch)
            us = _median(times)
            results.append((tile, us))
            print(f"tune: {name} {tile:>14s} {us:8.2f} us", file=log, flush=True)
    finally:
        os.environ.pop("CONV_I8_TILE", None)
        if saved is not None:
            os.environ["CONV_I8_TILE"] = saved
    results.sort(key=lambda r: r[1])
    key = (*c.image.dims, c.filter.dims[0], *c.filter.dims[2:], *c.pre, *c.post, *c.stride, *c.dilation,
           1 if lanes == "pixels" else 0)
    return results, key


def write_table(rows, device_name, path=INC):
    """rows: [(workload, key, [(tile, us), ...])]"""
    out = ["// Measured tile choices, written by int8_convolution_forward_amd/tune.py --write",
           f"// on {device_name}, {time.strftime('%Y-%m-%d')}: whole conv_fprop_i8_ws call, median of "
           f"{BATCHES} batches of",
           "// calls over rotating HBM-resident buffers.  Key: N, C, H, W, K, R, S, pre h/w, post h/w,",
           "// stride h/w, dilation h/w, output lanes (0 channels, 1 pixels).",
           ]
    for name, key, res in rows:
        if not res:
            continue
        others = ", ".join(f"{t} {us:.2f}" for t, us in res[1:])
        out.append(f"// {name}: {res[0][0]} {res[0][1]:.2f} us; then {others}")
        out.append("{" + ", ".join(str(int(k)) for k in key) + f', "{res[0][0]}"}},')
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", default="all")
    ap.add_argument("--write", action="store_true", help="rewrite csrc/tuned_tiles.inc")
    ap.add_argument("--out", default=INC, help="where --write puts the table")
    args = ap.parse_args(argv)

    import torch

    import workloads as wl

    names = list(wl.CASES) if args.workloads == "all" else args.workloads.split(",")
    rows = []
    for n in names:
        res, key = sweep(n)
        rows.append((n, key, res))
        best = f"{res[0][0]} {res[0][1]:.2f} us" if res else "none"
        print(f"{n}: fastest {best} of {len(res)} tiles", flush=True)
    if args.write:
        prop = torch.cuda.get_device_properties(0)
        write_table(rows, f"{prop.gcnArchName.split(':')[0]} with {prop.multi_processor_count} CUs", args.out)
        print(f"wrote {args.out}", flush=True)


if __name__ == "__main__":
    main()
