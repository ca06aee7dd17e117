"""Tile sweep: time every tile shape that applies to a problem, keep the fastest.

The cuDNN frontend tutorial page (its autotuning paragraph) builds every plan
the heuristics offer, times each one and ships the index of the fastest.  This
module does the same over the library's tile shapes (conv_i8_tile_names): for
each workload it forces each tile through CONV_I8_TILE, keeps the tiles the
planner accepts for that problem, times the whole conv_fprop_i8_ws call
(median of five batches over rotating HBM-resident buffer sets, so the
Infinity Cache cannot serve one call from the previous one) and reports the
table.  With --op wgrad it sweeps the weight gradient instead
(conv_wgrad_i8_ws, whose one forward call of the transposed operands takes
the tile; its split of the reduction stays the planner's).  With --write it
updates csrc/tuned_tiles.inc, the table the planner consults before its cost
model, keeping the rows of workloads not swept (rebuild the library
afterwards).

    python -m int8_convolution_forward_amd.tune [--workloads a,b] [--op fprop|wgrad|both] [--write]

Run it from the repository root on the GPU the table is for.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import re
import sys
import time

INC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tuned_tiles.inc")
BATCHES = 5


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _operands(c, op, dev, rotate_mb):
    """Rotating HBM-resident buffer sets [(a, b, y)] of strided views in the
    argument order of the timed entry: fprop (image, filter, out INT32),
    wgrad (image, loss INT8 shaped like the output, dW INT32 shaped like the
    filter)."""
    import torch

    import workloads as wl

    d = wl.make_inputs(c, c.seed_base)
    a0, _ = wl.to_device(d["x_storage"], c.image, dev)
    if op == "fprop":
        b0, _ = wl.to_device(d["w_storage"], c.filter, dev)
        b_spec, y_spec = c.filter, c.out
    else:
        g = torch.Generator().manual_seed(c.seed_base + 91)
        b0 = torch.randint(-128, 128, (c.out.storage_size,), dtype=torch.int8, generator=g).to(dev)
        b_spec, y_spec = c.out, wl.TensorSpec(c.filter.dims, c.filter.strides)
    set_bytes = a0.numel() + b0.numel() + 4 * y_spec.storage_size
    nsets = max(2, min(128, int(rotate_mb * 2**20 // set_bytes) + 1))
    sets = []
    for _ in range(nsets):
        a, b = a0.clone(), b0.clone()
        y = torch.empty(y_spec.storage_size, dtype=torch.int32, device=dev)
        sets.append((torch.as_strided(a, c.image.dims, c.image.strides, c.image.offset),
                     torch.as_strided(b, b_spec.dims, b_spec.strides, b_spec.offset),
                     torch.as_strided(y, y_spec.dims, y_spec.strides, y_spec.offset)))
    return sets


def table_key(c, op, lanes):
    """The table's key of a workload: op (0 forward, 1 weight gradient), the
    layer's N, C, H, W, K, R, S, padding, stride, dilation, and the output
    lanes (forward: the planned walk over channels 0 or pixels 1; weight
    gradient: dW channel-innermost 0 or not 1)."""
    if op == "wgrad":
        lanes = 0 if c.filter.strides[1] == 1 else 1
    else:
        lanes = 1 if lanes == "pixels" else 0
    return (0 if op == "fprop" else 1, *c.image.dims, c.filter.dims[0], *c.filter.dims[2:], *c.pre, *c.post,
            *c.stride, *c.dilation, lanes)


def sweep(name, op="fprop", calls_per_batch=200, warmup=300, rotate_mb=600.0, log=sys.stderr):
    """[(tile, us)] for every tile the planner accepts on workload `name`
    (op "fprop": conv_fprop_i8_ws; op "wgrad": conv_wgrad_i8_ws, whose one
    forward call takes the tile), fastest first, plus the table key."""
    import torch

    import int8_convolution_forward_amd as ci8
    import workloads as wl

    c = wl.case(name)
    dev = torch.device("cuda:0")
    sets = _operands(c, op, dev, rotate_mb)
    nsets = len(sets)
    params = ci8._params(c.pre, c.post, c.stride, c.dilation, None)
    geo = (c.pre, c.post, c.stride, c.dilation)
    if op == "fprop":
        plan = lambda s: ci8.conv_fprop_i8_plan(*s, *geo)
        wsize = lambda s: ci8.conv_fprop_i8_workspace_size(*s, *geo)
        fn, extra = ci8.lib.conv_fprop_i8_ws, ()
    else:
        plan = lambda s: ci8.conv_wgrad_i8_plan(*s, *geo)
        wsize = lambda s: ci8.conv_wgrad_i8_workspace_size(*s, *geo)
        fn, extra = ci8.lib.conv_wgrad_i8_ws, (ctypes.c_int32(0),)
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    saved = os.environ.pop("CONV_I8_TILE", None)
    results = []
    lanes = None
    if op == "wgrad" and ci8.plan_fields(plan(sets[0])).get("kernel") == "wgrad_in_place":
        # a gradient read in place by its own kernel: no tile to choose
        print(f"tune: {op} {name}: the in-place weight-gradient kernel, not swept", file=log, flush=True)
        if saved is not None:
            os.environ["CONV_I8_TILE"] = saved
        return [], None
    try:
        for tile in ci8.conv_i8_tile_names():
            os.environ["CONV_I8_TILE"] = tile
            f = ci8.plan_fields(plan(sets[0]))
            lanes = f.get("lanes")
            if f.get("tile") != tile:
                continue        # does not apply to this problem
            wsb = wsize(sets[0])
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            calls = [(ctypes.byref(ci8.desc(s[0])), ctypes.c_void_p(s[0].data_ptr()),
                      ctypes.byref(ci8.desc(s[1])), ctypes.c_void_p(s[1].data_ptr()),
                      ctypes.byref(ci8.desc(s[2])), ctypes.c_void_p(s[2].data_ptr()), *params, *extra,
                      ctypes.c_void_p(ws.data_ptr()) if wsb else None, ctypes.c_size_t(wsb), sh)
                     for s in sets]

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
            print(f"tune: {op} {name} {tile:>14s} {us:8.2f} us", file=log, flush=True)
    finally:
        os.environ.pop("CONV_I8_TILE", None)
        if saved is not None:
            os.environ["CONV_I8_TILE"] = saved
    results.sort(key=lambda r: r[1])
    return results, table_key(c, op, lanes)


_ROW = re.compile(r"^// (fprop|wgrad) (\S+): ")


def read_table(path=INC):
    """{(op, workload): (comment line, entry line)} of an existing table."""
    rows = {}
    try:
        lines = open(path).read().splitlines()
    except FileNotFoundError:
        return rows
    for i, line in enumerate(lines[:-1]):
        m = _ROW.match(line)
        if m and lines[i + 1].startswith("{"):
            rows[(m.group(1), m.group(2))] = (line, lines[i + 1])
    return rows


def write_table(rows, device_name, path=INC):
    """rows: [(op, workload, key, [(tile, us), ...])]; entries of the table
    already at `path` for other (op, workload) pairs are kept, and a pair
    swept with no tile to choose (key None) loses its entry."""
    table = read_table(path)
    for op, name, key, res in rows:
        if key is None:
            table.pop((op, name), None)
        if not res:
            continue
        others = ", ".join(f"{t} {us:.2f}" for t, us in res[1:])
        table[(op, name)] = (f"// {op} {name}: {res[0][0]} {res[0][1]:.2f} us; then {others}",
                             "{" + ", ".join(str(int(k)) for k in key) + f', "{res[0][0]}"}},')
    out = ["// Measured tile choices, written by int8_convolution_forward_amd/tune.py --write",
           f"// on {device_name}, {time.strftime('%Y-%m-%d')}: whole conv_fprop_i8_ws (fprop) or",
           f"// conv_wgrad_i8_ws (wgrad) call, median of {BATCHES} batches of calls over rotating",
           "// HBM-resident buffers.  Key: op (0 fprop, 1 wgrad), N, C, H, W, K, R, S of the layer,",
           "// pre h/w, post h/w, stride h/w, dilation h/w, lanes (fprop: output lanes walk",
           "// channels 0 or pixels 1; wgrad: dW channel-innermost 0 or not 1).",
           ]
    for op in ("fprop", "wgrad"):
        for (o, name), (comment, entry) in sorted(table.items()):
            if o == op:
                out += [comment, entry]
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workloads", default="all")
    ap.add_argument("--op", default="fprop", choices=("fprop", "wgrad", "both"))
    ap.add_argument("--write", action="store_true", help="rewrite csrc/tuned_tiles.inc")
    ap.add_argument("--out", default=INC, help="where --write puts the table")
    args = ap.parse_args(argv)

    import torch

    import workloads as wl

    names = list(wl.CASES) if args.workloads == "all" else args.workloads.split(",")
    rows = []
    for op in (("fprop", "wgrad") if args.op == "both" else (args.op,)):
        for n in names:
            res, key = sweep(n, op)
            rows.append((op, n, key, res))
            best = f"{res[0][0]} {res[0][1]:.2f} us" if res else "none"
            print(f"{op} {n}: fastest {best} of {len(res)} tiles", flush=True)
    if args.write:
        prop = torch.cuda.get_device_properties(0)
        write_table(rows, f"{prop.gcnArchName.split(':')[0]} with {prop.multi_processor_count} CUs", args.out)
        print(f"wrote {args.out}", flush=True)


if __name__ == "__main__":
    main()
