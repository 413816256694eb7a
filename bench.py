"""Benchmark of the gfx950 fp16/fp32-accumulate GEMM (one JSON line on stdout).

A step is one C = A B over the whole workload (default: 8192 x 8192 x 8192, A and B
uniform on [-0.5, 0.5), seed 3), with A and B already resident in HBM.  W warm-up steps,
then K timed steps bracketed by device synchronisation.  Per-launch durations come from
HIP events recorded on the stream the kernel is launched on (torch's current stream).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--tile T] [--group-m G] [--xcd-remap R] [--layout AB[C]]
                    [--layouts] [--dist D] [--vs-torch] [--no-cpu-baseline] [--floor]
                    [--mfma-ceiling [--mfma-shape S]]

`value` is TFLOP/s = 2 M N K K_steps / (timed wall time); `roofline.achieved` is
2 M N K / (mean per-launch event time), against the MI355X published dense fp16 matrix
peak of 2.5 PFLOP/s.  `cpu_baseline` times the CPU oracle (fp64 ascending-k sums, one
rounding) on the whole product of the same workload (about 3 s on a 16-thread host), using
all host threads it gets.
--all prints one extra JSON line per workload to stderr, with the device time per launch
from HIP-graph replays beside the per-launch event times.  --layout stores A, B (and C) row-
major ("n") or column-major ("t"), e.g. "nt" for B given as an N x K matrix; --layouts times
all eight storage orders (stderr).  --dist draws the operands from another distribution of
synthetic_inputs (e.g. "zeros" or "s(1/64)", which switch fewer bits in the matrix cores)
with the workload's shape and seed; `config.dist` names the one used.  After the timed region
the same launches run for 3 s while the XCD clocks and the socket power are sampled.
--floor only times, in HIP-graph replays, the launches that bound the small workloads from
below (an empty launch, K = 0, one workgroup on one panel).  --mfma-ceiling only times the
matrix-core rate probe: the 8192^3 GEMM's MFMAs from registers, with no memory traffic
(--mfma-shape 32x32x16: the same flops in the other fp16 MFMA shape, for comparison).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fp16-in/fp32-acc GEMM TFLOP/s at 8192³ on 1 MI355X; % of fp16 MFMA peak"
PEAK_TFLOPS = 2500.0          # MI355X published dense fp16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


from dense_gemm_f16f32_amd.build import kernel_source_hash, strip_comments  # noqa: E402,F401


def measured_traffic(workload: str, tile: int, group_m: int, remap: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when they
    were taken for another kernel source or launch configuration."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{workload}/tile{tile}/g{group_m}/remap{remap}"
    e = rec.get(key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


_DEVICE_OPERANDS = {}


def device_operands(torch, name, dist=None):
    """(A, B, C) device tensors of a workload (operands from `dist` instead of the workload's
    own distribution if given), generated once per process."""
    import numpy as np
    from synthetic_inputs import operands, workload

    key = (name, dist)
    if key not in _DEVICE_OPERANDS:
        _DEVICE_OPERANDS.clear()
        _, M, N, K, wdist, seed = workload(name)
        A, B = operands(M, N, K, dist or wdist, seed)
        _DEVICE_OPERANDS[key] = (torch.from_numpy(A.view(np.int16)).cuda(),
                                 torch.from_numpy(B.view(np.int16)).cuda(),
                                 torch.empty((M, N), dtype=torch.int16, device="cuda"))
    return _DEVICE_OPERANDS[key]


def layout_views(torch, A, B, C, layout):
    """A, B, C as views with the storage orders named by `layout` ("n" row-major, "t"
    column-major, for A, B and optionally C; the data are the same logical matrices)."""
    lay = (layout + "n")[:3]
    if lay[0] == "t":
        A = A.t().contiguous().t()
    if lay[1] == "t":
        B = B.t().contiguous().t()
    if lay[2] == "t":
        C = torch.empty((C.shape[1], C.shape[0]), dtype=C.dtype, device=C.device).t()
    return A, B, C


def time_workload(g, torch, name, steps, warmup, opts, layout="nn", dist=None):
    from synthetic_inputs import workload

    _, M, N, K, _, _ = workload(name)
    Ad, Bd, Cd = layout_views(torch, *device_operands(torch, name, dist), layout)
    rc, plan = g.gemm_f16f32_strided_plan(M, N, K, Ad.data_ptr(), *Ad.stride(), Bd.data_ptr(),
                                          *Bd.stride(), Cd.data_ptr(), *Cd.stride(),
                                          opts=opts or None)
    if rc != g.OK:
        raise g.GemmError(rc, "plan")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.matmul(Ad, Bd, Cd, **opts)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        g.matmul(Ad, Bd, Cd, **opts)
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in ev)      # ms
    flops = 2.0 * M * N * K
    mean_ms = sum(per) / len(per)
    return {
        "workload": name, "M": M, "N": N, "K": K, "layout": layout, "plan": plan,
        "value": flops * steps / wall / 1e12, "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_mean": mean_ms, "kernel_ms_median": per[len(per) // 2],
        "kernel_ms_min": per[0], "kernel_ms_p90": per[min(len(per) - 1, int(0.9 * len(per)))],
        "achieved_tflops": flops / (mean_ms * 1e-3) / 1e12,
    }


def graph_device_us(torch, fn, n=20, reps=5):
    """Device time per launch (us) of fn, from replays of a HIP graph of n launches: the host
    launch cost, which per-launch events see for kernels of a few microseconds, drops out."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
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
    return sorted(res)[len(res) // 2]


def time_torch(torch, name, steps, warmup, dist=None):
    """torch.matmul (the vendor BLAS) on the same fp16 operands, for context only."""
    from synthetic_inputs import workload

    _, M, N, K, wdist, _ = workload(name)
    Ad, Bd, _ = device_operands(torch, name, dist)
    a, b = Ad.view(torch.float16), Bd.view(torch.float16)
    for _ in range(warmup):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for s, e in ev:
        s.record()
        torch.matmul(a, b)
        e.record()
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in ev)
    mean = sum(per) / len(per)
    return {"context": "torch.matmul", "workload": name, "dist": dist or wdist,
            "tflops": round(2.0 * M * N * K / (mean * 1e-3) / 1e12, 1),
            "kernel_ms_median": round(per[len(per) // 2], 4)}


def vs_torch(g, torch, name, opts, dist=None, rounds=10, block=50, warm_s=3.0):
    """Interleaved A/B against torch.matmul (the vendor BLAS), for context only: after warm_s
    seconds of both, `rounds` rounds of one block of each (order alternating), per-launch HIP
    events; the median over rounds of each block's mean launch time."""
    import statistics
    from synthetic_inputs import workload

    _, M, N, K, wdist, _ = workload(name)
    Ad, Bd, Cd = device_operands(torch, name, dist)
    a, b = Ad.view(torch.float16), Bd.view(torch.float16)
    fns = {"library": lambda: g.matmul(Ad, Bd, Cd, **opts),
           "torch.matmul": lambda: torch.matmul(a, b)}
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            for fn in fns.values():
                fn()
        torch.cuda.synchronize()

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(block)]
        for s, e in ev:
            s.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in ev) / block

    res = {k: [] for k in fns}
    for r in range(rounds):
        for k in (list(fns) if r % 2 == 0 else list(fns)[::-1]):
            res[k].append(timed(fns[k]))
    out = {"ab": "interleaved", "workload": name, "dist": dist or wdist, "rounds": rounds,
           "block": block}
    for k, v in res.items():
        med = statistics.median(v)
        out[k] = {"ms_median": round(med, 5), "ms_min": round(min(v), 5),
                  "ms_max": round(max(v), 5),
                  "tflops": round(2.0 * M * N * K / (med * 1e-3) / 1e12, 1)}
    return out


def latency_floor(torch, g):
    """Device time per launch in HIP-graph replays of launches that bound the two small
    workloads from below: a one-element fill (torch's, the launch alone), the library with
    K = 0 (launch and store of a 512 x 512 C), one workgroup on one 64-deep panel (32 x 32 x
    64: the launch, one load round trip, the store), one panel on 128 workgroups (512 x 512 x
    64), and the two small workloads themselves.  One JSON line each on stderr."""
    import numpy as np
    from synthetic_inputs import operands

    one = torch.empty(1, dtype=torch.float32, device="cuda")
    us = graph_device_us(torch, lambda: one.zero_(), n=50)
    print(json.dumps({"floor": "fill of 1 element (torch)", "graph_us_per_launch": round(us, 3)}),
          file=sys.stderr, flush=True)
    for M, N, K, opts, what in ((512, 512, 0, {}, "K = 0: launch and store of C"),
                                (32, 32, 64, {}, "one workgroup, one panel"),
                                (512, 512, 64, {}, "one panel, 128 workgroups"),
                                (512, 512, 512, {}, "the 512^3 workload"),
                                (1024, 768, 128, {"tile": g.TILE_128x64x64, "group_m": 2},
                                 "the 1024 x 768 x 128 workload")):
        A, B = operands(M, N, K, "u(-0.5,0.5)", 0)
        Ad = torch.from_numpy(A.view(np.int16)).cuda()
        Bd = torch.from_numpy(B.view(np.int16)).cuda()
        Cd = torch.empty((M, N), dtype=torch.int16, device="cuda")
        us = graph_device_us(torch, lambda: g.matmul(Ad, Bd, Cd, **opts), n=50)
        print(json.dumps({"floor": what, "M": M, "N": N, "K": K,
                          "graph_us_per_launch": round(us, 3)}), file=sys.stderr, flush=True)


MFMA_SHAPES = {"16x16x32": 0, "32x32x16": 1}


def mfma_ceiling(torch, dist, steps, warmup, clocks, shape="16x16x32"):
    """The matrix cores alone (dense_gemm_f16f32_amd/libmfma_ceiling.so, the rate probe):
    each launch issues the 8192^3 GEMM's 2^26 v_mfma_f32_16x16x32_f16 on the GEMM's grid and
    in its operand pattern, from registers only, on operands uniform on [-0.5, 0.5) or all
    +0 (dist "zeros").  With shape "32x32x16" it issues the same flops as 2^25
    v_mfma_f32_32x32x16_f16 instead.  Timed like the GEMM (W warm-up launches, K timed ones,
    per-launch events) and followed by the same clock and power sampling; one JSON line on
    stdout."""
    import ctypes

    if dist not in (None, "zeros", "u(-0.5,0.5)"):
        raise SystemExit("--mfma-ceiling takes --dist zeros or the default u(-0.5,0.5)")
    lib = ctypes.CDLL(os.path.join(ROOT, "dense_gemm_f16f32_amd", "libmfma_ceiling.so"))
    f = lib.mfma_ceiling_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_uint32, ctypes.c_void_p]
    if shape not in MFMA_SHAPES:
        raise SystemExit("--mfma-shape takes " + " or ".join(MFMA_SHAPES))
    blocks, iters = 256, 512        # 1024 wavefronts x 512 x 128 MFMAs of 16x16x32 = 2^26
    flops = blocks * 4 * iters * 128 * (2 * 16 * 16 * 32)
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = f(out.data_ptr(), blocks, iters, MFMA_SHAPES[shape], 1 if dist == "zeros" else 0, 3,
               stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mfma_ceiling_launch: hipError {rc}")

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(ms) / len(ms)
    achieved = flops / (mean * 1e-3) / 1e12
    res = {"probe": "mfma_ceiling", "mfma": f"v_mfma_f32_{shape}_f16",
           "dist": dist or "u(-0.5,0.5)",
           "mfmas_per_launch": 1 << 26 if shape == "16x16x32" else 1 << 25,
           "steps": steps, "warmup": warmup, "value": round(flops * steps / wall / 1e12, 2),
           "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
           "frac": round(achieved / PEAK_TFLOPS, 4),
           "kernel_ms": {"mean": round(mean, 5), "median": round(ms[len(ms) // 2], 5),
                         "min": round(ms[0], 5)}}
    if clocks:
        c = sample_clocks(None, torch, launch)
        if c:
            peak = 256 * 4096 * c["median"] * 1e6 / 1e12
            res.update(sclk_mhz=c, peak_at_sclk=round(peak, 1),
                       frac_at_sclk=round(achieved / peak, 4))
    print(json.dumps(res), flush=True)


def copy_calibration(torch, mib, steps):
    """A plain device copy of known size, timed; profiled with the same HBM counters as the
    GEMM it gives the factor between counter readings and bytes actually moved."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": steps,
                      "GB_per_s": round(2 * n / dt / 1e9, 1)}), flush=True)


def parse_smi(text):
    """(GFX clock of every XCD in MHz, socket power in W or None) from the text of
    `amd-smi metric -c -p`: the CLK line of each GFX_<n> block, and the SOCKET_POWER line."""
    import re
    clocks, in_gfx, power = [], False, None
    for line in text.splitlines():
        if re.match(r"\s*GFX_\d+:\s*$", line):
            in_gfx = True
            continue
        m = re.match(r"\s*CLK:\s*(\d+)", line)
        p = re.match(r"\s*SOCKET_POWER:\s*([\d.]+)", line)
        if in_gfx and m:
            clocks.append(int(m.group(1)))
            in_gfx = False
        elif p:
            power = float(p.group(1))
        elif line.strip().endswith(":"):
            in_gfx = False
    return clocks, power


def smi_sample():
    """Current XCD clocks and socket power (parse_smi of one `amd-smi metric -c -p`; [] and
    None if amd-smi is unavailable)."""
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-c", "-p"], capture_output=True, text=True,
                             timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return [], None
    return parse_smi(out)


def sample_clocks(g, torch, fn, seconds=3.0):
    """Runs fn back to back for `seconds` (untimed, after the timed region) while sampling the
    XCD clocks and the socket power; returns the 5th percentile, median and 95th percentile
    in MHz over all samples and XCDs, and the median socket power in W, or None."""
    import threading
    samples, powers, done = [], [], threading.Event()

    def poll():
        while not done.is_set():
            c, pw = smi_sample()
            samples.extend(c)
            if pw is not None:
                powers.append(pw)
            time.sleep(0.2)

    if not smi_sample()[0]:
        return None
    for _ in range(20):          # the clocks ramp up before sampling starts
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    for _ in range(20):          # work is queued before the first sample is taken
        fn()
    prev = torch.cuda.Event()
    prev.record()
    t_end = time.perf_counter() + seconds
    th.start()
    while True:
        for _ in range(20):
            fn()
        ev = torch.cuda.Event()
        ev.record()
        if prev is not None:     # one batch stays queued, so the GPU never idles
            prev.synchronize()
        prev = ev
        if time.perf_counter() >= t_end:
            done.set()           # the poller may be inside a sample: keep the GPU busy
            if not th.is_alive():  # until it has returned, so no sample sees it idle
                break
    th.join()
    torch.cuda.synchronize()
    if not samples:
        return None
    samples.sort()
    q = lambda f: samples[min(len(samples) - 1, int(f * len(samples)))]
    # an XCD occasionally reads a few hundred MHz for an instant; percentiles keep such
    # outliers from standing for the run
    powers.sort()
    return {"p05": q(0.05), "median": q(0.5), "p95": q(0.95), "samples": len(samples),
            "socket_power_w": powers[len(powers) // 2] if powers else None}


def cpu_all():
    """The oracle on every workload (one JSON line each): the whole product on all threads,
    plus one thread on the two small workloads.  Records the host CPU."""
    import numpy as np
    import oracle
    from synthetic_inputs import WORKLOADS, operands

    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    oracle.lib()
    for name, M, N, K, dist, seed in WORKLOADS:
        A, B = operands(M, N, K, dist, seed)
        rows = M
        Ab = A
        res = {"workload": name, "rows": rows, "N": N, "K": K, "cpu": model,
               "nproc": os.cpu_count()}
        t0 = time.perf_counter()
        oracle.gemm(Ab, B)
        dt = time.perf_counter() - t0
        res["all_threads"] = {"s": round(dt, 4), "threads": oracle.num_threads(),
                              "GFLOP/s": round(2.0 * rows * N * K / dt / 1e9, 2)}
        if M * N * K <= 1 << 31:
            dt1 = _oracle_single_thread_seconds(Ab, B)
            res["single_thread"] = {"s": round(dt1, 4), "threads": 1,
                                    "GFLOP/s": round(2.0 * rows * N * K / dt1 / 1e9, 2)}
        print(json.dumps(res), flush=True)


def _oracle_single_thread_seconds(A, B):
    """Seconds of one oracle GEMM on one host thread, timed inside a child process (OpenMP's
    thread count is fixed once the library is loaded in this one)."""
    import subprocess
    import tempfile

    import numpy as np
    with tempfile.TemporaryDirectory() as d:
        pa, pb = os.path.join(d, "a.npy"), os.path.join(d, "b.npy")
        np.save(pa, A)
        np.save(pb, B)
        code = ("import sys, time, numpy as np; sys.path.insert(0, %r); import oracle; "
                "a, b = np.load(%r), np.load(%r); oracle.lib(); t = time.perf_counter(); "
                "oracle.gemm(a, b); print(time.perf_counter() - t)" % (ROOT, pa, pb))
        env = dict(os.environ, OMP_NUM_THREADS="1")
        out = subprocess.run([sys.executable, "-c", code], env=env, check=True,
                             capture_output=True, text=True).stdout
    return float(out.strip().splitlines()[-1])


def cpu_baseline(name: str, rows: int = 0):
    """The oracle's rate on the first `rows` rows of the workload's C (0: all of it)."""
    import numpy as np
    import oracle
    from synthetic_inputs import operands, workload

    _, M, N, K, dist, seed = workload(name)
    A, B = operands(M, N, K, dist, seed)
    rows = M if rows <= 0 else min(rows, M)
    Ab = A if rows == M else np.ascontiguousarray(A[:rows])
    del A
    oracle.lib()
    t0 = time.perf_counter()
    oracle.gemm(Ab, B)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"the whole {M} x {N} x {K} product of {name}" if rows == M else
                       f"rows 0..{rows - 1} of C ({rows} x {N} outputs, K = {K}) of {name}")
                      + f", {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gemm8192_u")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=0)
    ap.add_argument("--force-generic", type=int, default=0)
    ap.add_argument("--layout", default="nn",
                    help="storage of A, B[, C]: n = row-major, t = column-major (e.g. nt)")
    ap.add_argument("--layouts", action="store_true",
                    help="time every storage order of A, B and C (stderr)")
    ap.add_argument("--dist", default=None,
                    help="operand distribution instead of the workload's (e.g. zeros, s(1/64))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time GROUP_SIZE_M in 1..32 with the XCD permutation on and off (stderr)")
    ap.add_argument("--vs-torch", action="store_true",
                    help="interleaved A/B against torch.matmul after a warm-up (stderr)")
    ap.add_argument("--torch", action="store_true",
                    help="also time torch.matmul on the same operands (stderr, context only; "
                         "it runs before the library's timed steps, so --vs-torch compares)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the 3 s clock sampling after the timed region")
    ap.add_argument("--cpu-all", action="store_true",
                    help="only time the CPU oracle on every workload (no GPU)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the matrix-core rate probe (the GEMM's MFMAs from "
                         "registers, no memory traffic) on --dist zeros or the default data")
    ap.add_argument("--mfma-shape", default="16x16x32",
                    help="with --mfma-ceiling: 16x16x32 (the GEMM's MFMAs) or 32x32x16")
    ap.add_argument("--floor", action="store_true",
                    help="only time, in HIP-graph replays, launches that bound the small "
                         "workloads from below (stderr)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only time a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GEMM runs on a single MI355X and the library "
              "has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.cpu_all:
        cpu_all()
        return

    import torch
    import dense_gemm_f16f32_amd as g
    from synthetic_inputs import WORKLOADS, workload

    torch.cuda.set_device(0)
    if args.copy_mib:
        copy_calibration(torch, args.copy_mib, args.steps)
        return
    if args.floor:
        latency_floor(torch, g)
        return
    if args.mfma_ceiling:
        mfma_ceiling(torch, args.dist, args.steps, args.warmup, not args.no_clocks,
                     args.mfma_shape)
        return
    opts = {k: v for k, v in (("tile", args.tile), ("group_m", args.group_m),
                              ("xcd_remap", args.xcd_remap),
                              ("force_generic", args.force_generic)) if v}

    if args.all:
        for w in WORKLOADS:
            small = w[1] * w[2] * w[3] < 1 << 31
            r = time_workload(g, torch, w[0], 1000 if small else 50, 10, opts)
            r["frac_of_peak"] = r["achieved_tflops"] / PEAK_TFLOPS
            Ad, Bd, Cd = device_operands(torch, w[0])
            us = graph_device_us(torch, lambda: g.matmul(Ad, Bd, Cd, **opts),
                                 n=50 if small else 5)
            r["graph_us_per_launch"] = round(us, 3)
            r["graph_tflops"] = round(2.0 * w[1] * w[2] * w[3] / us / 1e6, 1)
            print(json.dumps(r), file=sys.stderr, flush=True)

    if args.sweep:
        # interleaved: 4 rounds over all (G, permutation) pairs, alternating direction, each
        # a block of `steps` event-timed launches; the median of the block medians per pair
        # (the chip's power state drifts over a sweep)
        pairs = [(G, remap) for G in (1, 2, 4, 8, 16, 32) for remap in (1, 2)]
        blocks = {pr: [] for pr in pairs}
        for rnd in range(4):
            for G, remap in (pairs if rnd % 2 == 0 else pairs[::-1]):
                o = dict(opts, group_m=G, xcd_remap=remap)
                rr = time_workload(g, torch, args.workload, args.steps,
                                   args.warmup if rnd == 0 else 2, o)
                blocks[(G, remap)].append(rr["kernel_ms_median"])
        _, M, N, K, _, _ = workload(args.workload)
        for (G, remap), v in blocks.items():
            med = sorted(v)[len(v) // 2]
            print(json.dumps({"workload": args.workload, "group_m": G,
                              "xcd_remap": remap == 1, "rounds": len(v),
                              "kernel_ms_median": round(med, 4),
                              "tflops": round(2.0 * M * N * K / (med * 1e-3) / 1e12, 1)}),
                  file=sys.stderr, flush=True)
    if args.layouts:
        for lay in ("nn", "nt", "tn", "tt", "nnt", "ntt", "tnt", "ttt"):
            rr = time_workload(g, torch, args.workload, args.steps, args.warmup, opts, lay)
            print(json.dumps({"workload": args.workload, "layout": lay,
                              "tflops": round(rr["achieved_tflops"], 1),
                              "kernel_ms_median": round(rr["kernel_ms_median"], 4)}),
                  file=sys.stderr, flush=True)
    if args.torch:
        print(json.dumps(time_torch(torch, args.workload, args.steps, args.warmup, args.dist)),
              file=sys.stderr, flush=True)
    if args.vs_torch:
        print(json.dumps(vs_torch(g, torch, args.workload, opts, args.dist)), file=sys.stderr,
              flush=True)

    r = time_workload(g, torch, args.workload, args.steps, args.warmup, opts, args.layout,
                      args.dist)
    plan = r["plan"]
    clocks = None
    if not args.no_clocks:
        Ad, Bd, Cd = layout_views(torch, *device_operands(torch, args.workload, args.dist),
                                  args.layout)
        clocks = sample_clocks(g, torch, lambda: g.matmul(Ad, Bd, Cd, **opts))
    # the counters were taken on the workload's own operands in row-major storage
    traffic = (measured_traffic(args.workload, plan["tile"], plan["group_m"], plan["xcd_remap"])
               if args.layout == "nn" and args.dist is None else None)
    out = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "M": r["M"], "N": r["N"], "K": r["K"],
            "dist": args.dist or workload(args.workload)[4],
            "accumulate": "f32", "layout": args.layout,
            "path": ["dma", "generic"][plan["path"]],
            "tile": f"{plan['bm']}x{plan['bn']}x{plan['bk']}", "tile_id": plan["tile"],
            "threads": plan["threads"], "group_m": plan["group_m"],
            "xcd_remap": plan["xcd_remap"], "workgroups": plan["num_programs"],
            "launches": plan["launches"],
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(r["achieved_tflops"], 2),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(r["achieved_tflops"] / PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms": {k: round(r["kernel_ms_" + k], 5) for k in ("mean", "median", "min",
                                                                      "p90")},
            # XCD clocks (and socket power) while the same launches run back to back (3 s after
            # the timed region) and the dense fp16 peak at their median: 256 CUs x 4096 flop/clk
            # x f
            "sclk_mhz": clocks,
            "peak_at_sclk": (round(256 * 4096 * clocks["median"] * 1e6 / 1e12, 1)
                             if clocks else None),
            "frac_at_sclk": (round(r["achieved_tflops"] /
                                   (256 * 4096 * clocks["median"] * 1e6 / 1e12), 4)
                             if clocks else None),
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(args.workload),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
