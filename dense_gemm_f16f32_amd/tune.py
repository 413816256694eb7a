"""Offline sweep of tile configuration and GROUP_SIZE_M per shape class (runs on the GPU).

The launch grid of a GEMM depends on its tile shape, and which tile (and which group size)
is fastest depends on the problem's shape: the tutorial that the grouped order comes from
leaves the block sizes to an autotuner keyed on M, N and K.  This script is that autotuner,
run once, offline: for every shape class of a log2 grid it times each tile configuration
of the library (forced through gemm_f16f32_ex options), then GROUP_SIZE_M in 1..32 with the
XCD permutation on and off for the winner when the grid is large enough for the order to
matter, and writes the winners as a C table (csrc/tune_table.inc, headed by the kernel
source hash it was measured at) that the library's planner looks up by rounded log2 of
(M, N, K).

Each timing is the device time per launch of a HIP graph holding n back-to-back launches on
resident operands (uniform on [-0.5, 0.5), row-major, leading dimension = row length), so
host launch overhead does not enter.  The chip's power state drifts by several percent over a
sweep, so every shape is timed in a forward and a reverse pass over the tiles (averaged), and
tiles within 5 % of the fastest are timed again in six interleaved rounds and compared by
median.  Every forced configuration must also reproduce the first
configuration's bits (all tiles add the same MFMA k steps per element).

    python -m dense_gemm_f16f32_amd.tune [--out PATH] [--quick] [--k K,...] [--json PATH]
    python -m dense_gemm_f16f32_amd.tune --from-json a.json,b.json,...   (merge partial sweeps)

`--split-sweep` instead times split K (gemm_f16f32_strided_ws with split_k = S, the tile
chosen by the planner for each slice shape) for S in 1, 2, 4, ..., 32 and the automatic
choice, on thin and deep shapes, and prints one JSON line per shape: the data behind the
planner's automatic split rule (`--shapes` and `--splits` narrow it).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import dense_gemm_f16f32_amd as g  # noqa: E402

MN_GRID = [32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]
K_GRID = [64, 128, 256, 512, 1024, 2048, 4096, 8192]
GROUPS = [1, 2, 4, 8, 16, 32]
MARGIN = 0.03      # a new choice must be this much faster than the current one (one sweep)
CLOSE = 0.05       # tiles within this of the fastest are re-timed in interleaved rounds
AB_ROUNDS = 6
AB_MARGIN = 0.01   # ... and must then beat the current choice by this much (median)
TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tune_table.inc")


def graph_time_us(torch, fn, target_us=3000.0, reps=3):
    """Median over `reps` replays of a graph of n launches of fn, per launch (us)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        torch.cuda.synchronize()
        est = max(a.elapsed_time(b) * 1e3, 1.0)
    torch.cuda.current_stream().wait_stream(s)
    n = int(max(3, min(64, target_us / est)))
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(n):
            fn()
    gr.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        gr.replay()
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) * 1e3 / n)
    del gr
    return sorted(res)[len(res) // 2]


def programs(M, N, tile):
    bm, bn = g.TILES[tile][:2]
    return -(-M // bm) * -(-N // bn)


def tune_shape(torch, M, N, K, quick=False):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M * 1000003 + N * 1009 + K)
    A = (torch.rand((M, K), device="cuda", generator=gen) - 0.5).half().view(torch.int16)
    B = (torch.rand((K, N), device="cuda", generator=gen) - 0.5).half().view(torch.int16)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    split_off = dict(split_edges=g.SPLIT_OFF)
    # Two passes, forward and reverse tile order, averaged: the chip heats up (and slows
    # down) over a pass, which would otherwise favour whichever tile is timed first.
    tiles = [t for t in sorted(g.TILES) if not (quick and programs(M, N, t) > 4096)]
    passes, ref = {t: [] for t in tiles}, None
    for order in (tiles, tiles[::-1]):
        for tile in order:
            opts = dict(tile=tile, **split_off)
            passes[tile].append(graph_time_us(torch, lambda: g.matmul(A, B, C, **opts)))
            bits = C.cpu()
            if ref is None:
                ref = bits
            elif not torch.equal(bits, ref):
                raise RuntimeError(f"tile {tile} changed the result at {M}x{N}x{K}")
    times = {t: sum(v) / len(v) for t, v in passes.items()}
    auto = graph_time_us(torch, lambda: g.matmul(A, B, C))
    # the library's current choice (table or heuristic) stays unless another tile is clearly
    # faster in this same sweep: timings of large shapes move by several percent with the
    # chip's power state, and a table that flips on noise helps nobody
    rc, cur = g.gemm_f16f32_plan(M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), K, N, N,
                                 opts=split_off)
    current = cur["tile"]
    best = min(times, key=times.get)
    # Close contenders (within CLOSE of the fastest, plus the current choice if it is one)
    # are re-timed in interleaved rounds, which cancels the drift of the chip's power state
    # between the sweep's tiles; the current choice then stays unless another one is at least
    # AB_MARGIN faster by median.
    close = [t for t in sorted(times, key=times.get) if times[t] <= (1 + CLOSE) * times[best]]
    close = close[:3] + ([current] if current in times and current not in close[:3]
                         and times[current] <= (1 + CLOSE) * times[best] else [])
    ab = {}
    if len(close) > 1:
        fns = {t: (lambda t=t: g.matmul(A, B, C, tile=t, **split_off)) for t in close}
        runs = {t: [] for t in close}
        for r in range(AB_ROUNDS):
            order = close[r % len(close):] + close[:r % len(close)]
            for t in order:
                runs[t].append(graph_time_us(torch, fns[t], target_us=1500.0))
        ab = {t: sorted(v)[len(v) // 2] for t, v in runs.items()}
        best = min(ab, key=ab.get)
        if current in ab and ab[best] > (1.0 - AB_MARGIN) * ab[current]:
            best = current
    elif current in times and times[best] > (1.0 - MARGIN) * times[current]:
        best = current
    # GROUP_SIZE_M and the XCD permutation (on: key "G", off: key "Gx"), for grids large
    # enough for the order to matter: two passes over the 12 orders, then interleaved rounds
    # among the closest; the tile's default (its G, permutation on) stays unless another
    # order is clearly faster in those rounds
    group, remap, group_times, group_ab = 0, 0, {}, {}
    if programs(M, N, best) >= 128:
        rc, info = g.gemm_f16f32_plan(M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), K, N,
                                      N, opts=dict(tile=best))
        default_key = str(info["group_m"])
        keys = [f"{G}{x}" for G in GROUPS for x in ("", "x")]
        fns = {k: (lambda k=k: g.matmul(A, B, C, tile=best, group_m=int(k.rstrip("x")),
                                        xcd_remap=g.REMAP_OFF if k.endswith("x") else
                                        g.REMAP_ON, **split_off)) for k in keys}
        runs = {k: [] for k in keys}
        for r in range(2):
            for k in (keys if r % 2 == 0 else keys[::-1]):
                runs[k].append(graph_time_us(torch, fns[k], target_us=1500.0))
        group_times = {k: sum(v) / len(v) for k, v in runs.items()}
        gbest = min(group_times, key=group_times.get)
        # As for the tiles: orders within CLOSE of the fastest (and the default) are re-timed
        # in interleaved rounds; the default stays unless another is AB_MARGIN faster there.
        close = [k for k in sorted(group_times, key=group_times.get)
                 if group_times[k] <= (1 + CLOSE) * group_times[gbest]][:4]
        if default_key not in close:
            close.append(default_key)
        if len(close) > 1:
            gruns = {k: [] for k in close}
            for r in range(AB_ROUNDS):
                for k in close[r % len(close):] + close[:r % len(close)]:
                    gruns[k].append(graph_time_us(torch, fns[k], target_us=1500.0))
            group_ab = {k: sorted(v)[len(v) // 2] for k, v in gruns.items()}
            gbest = min(group_ab, key=group_ab.get)
            if gbest != default_key and \
                    group_ab[gbest] < (1.0 - AB_MARGIN) * group_ab[default_key]:
                group, remap = int(gbest.rstrip("x")), (2 if gbest.endswith("x") else 0)
    return {"M": M, "N": N, "K": K, "best_tile": best, "group_m": group, "remap": remap,
            "current": current,
            "us": {str(k): round(v, 2) for k, v in times.items()},
            "ab_us": {str(k): round(v, 2) for k, v in ab.items()},
            "group_us": {str(k): round(v, 2) for k, v in group_times.items()},
            "group_ab_us": {str(k): round(v, 2) for k, v in group_ab.items()},
            "auto_us": round(auto, 2)}


SPLIT_SHAPES = [(32, 32), (64, 64), (128, 128), (256, 256), (512, 512), (1024, 1024),
                (2048, 2048), (64, 4096), (4096, 64), (256, 2048), (128, 8192), (4095, 1)]
SPLIT_K = [1024, 2048, 4096, 8192]
SPLITS = [1, 2, 4, 8, 16, 32]


def split_sweep(torch, shapes=None, splits=None):
    """Device time per call (us) of each split count and of the automatic choice, over the
    grid SPLIT_SHAPES x SPLIT_K or the given (M, N, K) list; `splits` restricts the split
    counts (SPLIT_K_AUTO for the automatic choice)."""
    ws = torch.empty(600 << 20, dtype=torch.uint8, device="cuda")
    if shapes is None:
        shapes = [(M, N, K) for M, N in SPLIT_SHAPES for K in SPLIT_K]
    for M, N, K in shapes:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(M * 1000003 + N * 1009 + K)
        A = (torch.rand((M, K), device="cuda", generator=gen) - 0.5).half()
        B = (torch.rand((K, N), device="cuda", generator=gen) - 0.5).half()
        C = torch.empty((M, N), dtype=torch.half, device="cuda")
        row = {"M": M, "N": N, "K": K}
        for S in (splits or SPLITS + [g.SPLIT_K_AUTO]):
            rc, info = g.gemm_f16f32_strided_plan(M, N, K, A.data_ptr(), K, 1, B.data_ptr(),
                                                  N, 1, C.data_ptr(), N, 1,
                                                  opts=dict(split_k=S))
            if rc != g.OK:
                raise RuntimeError(g.gemm_f16f32_strerror(rc))
            if S > 1 and info["splits"] < 2:
                continue
            us = graph_time_us(torch, lambda: g.matmul(A, B, C, workspace=ws, split_k=S))
            key = "auto" if S == g.SPLIT_K_AUTO else str(S)
            row[key] = {"us": round(us, 2), "tile": info["tile"],
                        "splits": info["splits"], "grid": info["grid"]}
        print(json.dumps(row), flush=True)


def write_table(path, results, device, source_hash):
    lines = [
        "// Tile configuration and GROUP_SIZE_M per shape class, written by",
        "// dense_gemm_f16f32_amd/tune.py from device-time sweeps on " + device + ",",
        f"// kernel source hash {source_hash} (build.kernel_source_hash at the time of the sweep).",
        "// Key: rounded log2 of M, N (32 .. 8192) and K (64 .. 8192); group 0 = the tile's",
        "// default; remap 0 = XCD permutation on (default), 2 = off.  Columns: log2 M, log2 N,",
        "// log2 K, tile, group, remap; the comment gives the chosen configuration's time and",
        "// the time of the choice it replaced (same sweep), us.",
    ]
    for r in results:
        lm, ln, lk = (int(round(math.log2(r[x]))) for x in ("M", "N", "K"))
        times = r.get("ab_us") or {}
        if str(r["best_tile"]) not in times or str(r.get("current")) not in times:
            times = r["us"]
        best_us = times[str(r["best_tile"])]
        remap = r.get("remap", 0)
        if r["group_m"]:
            best_us = r["group_us"][str(r["group_m"]) + ("x" if remap == 2 else "")]
        was = times.get(str(r.get("current")), r["auto_us"])
        lines.append(f"{{{lm}, {ln}, {lk}, {r['best_tile']}, {r['group_m']}, {remap}}},"
                     f"  // {r['M']}x{r['N']}x{r['K']}: {best_us} (was {was})")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=TABLE, help="table to write (C rows)")
    ap.add_argument("--json", default=None, help="also write every timing as JSON here")
    ap.add_argument("--quick", action="store_true", help="skip grids above 4096 workgroups")
    ap.add_argument("--from-json", default=None,
                    help="only rewrite the table from JSON files of earlier sweeps (comma-"
                         "separated; their shape classes are merged)")
    ap.add_argument("--k", default=None,
                    help="sweep only these K values of the grid (comma-separated); with "
                         "--json, the partial results can be merged with --from-json")
    ap.add_argument("--split-sweep", action="store_true",
                    help="time split K per split count instead (no table is written)")
    ap.add_argument("--shapes", default=None,
                    help="with --split-sweep: comma-separated MxNxK list instead of the grid")
    ap.add_argument("--splits", default=None,
                    help="with --split-sweep: comma-separated split counts, 'auto' for the "
                         "automatic choice (default: 1, 2, 4, 8, 16, 32, auto)")
    args = ap.parse_args()
    if args.split_sweep:
        import torch
        torch.cuda.set_device(0)
        shapes = None
        if args.shapes:
            shapes = [tuple(int(x) for x in sh.split("x")) for sh in args.shapes.split(",")]
        splits = None
        if args.splits:
            splits = [g.SPLIT_K_AUTO if x == "auto" else int(x) for x in args.splits.split(",")]
        split_sweep(torch, shapes, splits)
        return
    if args.from_json:
        results, devices, hashes = [], set(), set()
        for path in args.from_json.split(","):
            with open(path) as f:
                rec = json.load(f)
            results += rec["results"]
            devices.add(rec["device"])
            hashes.add(rec.get("source_hash", "unknown"))
        if len(hashes) != 1:
            raise SystemExit(f"sweeps of different kernel sources: {sorted(hashes)}")
        results.sort(key=lambda r: (r["K"], r["M"], r["N"]))
        write_table(args.out, results, " / ".join(sorted(devices)), hashes.pop())
        print(f"wrote {args.out} ({len(results)} shape classes)")
        return
    import torch

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    device = f"{props.name} ({getattr(props, 'gcnArchName', 'gfx950').split(':')[0]}, " \
             f"{props.multi_processor_count} CUs)"
    from dense_gemm_f16f32_amd.build import kernel_source_hash
    source_hash = kernel_source_hash()
    results = []
    t0 = time.time()
    k_grid = [int(k) for k in args.k.split(",")] if args.k else K_GRID
    for K in k_grid:
        for M in MN_GRID:
            for N in MN_GRID:
                r = tune_shape(torch, M, N, K, args.quick)
                results.append(r)
                print(json.dumps({k: r[k] for k in ("M", "N", "K", "best_tile", "group_m",
                                                    "auto_us")}
                                 | {"best_us": r["us"][str(r["best_tile"])],
                                    "elapsed_s": round(time.time() - t0, 1)}), flush=True)
    if not args.k:
        write_table(args.out, results, device, source_hash)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"device": device, "source_hash": source_hash, "results": results}, f)
    print(f"{'wrote ' + args.out if not args.k else 'swept'} ({len(results)} shape classes)",
          flush=True)


if __name__ == "__main__":
    main()
