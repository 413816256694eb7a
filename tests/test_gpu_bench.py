"""bench.py end to end on the GPU: a short run prints one JSON line with the fields and types
the benchmark contract names, consistent with each other (value from the timed steps, the
roofline from per-launch event times, frac = achieved / peak)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("extra", [[], ["--dist", "zeros", "--workload", "gemm4096_u"]],
                         ids=["default", "zeros-4096"])
def test_bench_line_follows_the_contract(extra):
    out = run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-clocks", *extra)
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(out[key], typ), key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["unit"] == "TFLOP/s" and out["higher_is_better"] is True
    assert out["vs_baseline"] is None and out["cpu_baseline"] is None
    cfg = out["config"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    assert abs(out["value"] - 2 * M * N * K / (out["ms_per_step"] * 1e-3) / 1e12) \
        <= 1e-3 * out["value"] + 0.01
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-4
    assert 0 < roof["frac"] < 1
    if extra:
        assert cfg["dist"] == "zeros" and (M, N, K) == (4096, 4096, 4096)
        assert roof["traffic"] is None          # the counters were taken on other operands
    else:
        assert cfg["dist"] == "u(-0.5,0.5)" and (M, N, K) == (8192, 8192, 8192)
        assert cfg["workload"] == "gemm8192_u" and cfg["tile"] == "256x256x64"
        assert roof["traffic"] is None or roof["traffic"] > 2 * (M * K + K * N + M * N)


def test_vs_torch_reports_both_sides():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--vs-torch",
                        "--workload", "gemm4096_u", "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline", "--no-clocks"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    ab = [json.loads(ln) for ln in r.stderr.splitlines() if ln.startswith('{"ab"')]
    assert len(ab) == 1, r.stderr[-2000:]
    ab = ab[0]
    assert ab["workload"] == "gemm4096_u" and ab["rounds"] == 10 and ab["block"] == 50
    for side in ("library", "torch.matmul"):
        t = ab[side]
        assert 0 < t["ms_min"] <= t["ms_median"] <= t["ms_max"]
        assert abs(t["tflops"] - 2 * 4096 ** 3 / (t["ms_median"] * 1e-3) / 1e12) < 0.1 + 1e-3 * t["tflops"]


@pytest.mark.parametrize("shape", ["16x16x32", "32x32x16"])
@pytest.mark.parametrize("dist", [[], ["--dist", "zeros"]], ids=["u", "zeros"])
def test_mfma_ceiling_probe_reports_its_rate(dist, shape):
    """bench.py --mfma-ceiling: the rate probe's MFMAs per launch (2^26 of 16x16x32 or the same
    flops as 2^25 of 32x32x16), a rate below the nominal peak, and frac = achieved / peak."""
    out = run_bench("--mfma-ceiling", "--mfma-shape", shape, "--steps", "3", "--warmup", "1",
                    "--no-clocks", *dist)
    assert out["probe"] == "mfma_ceiling" and out["mfma"] == f"v_mfma_f32_{shape}_f16"
    assert out["mfmas_per_launch"] == (1 << 26 if shape == "16x16x32" else 1 << 25)
    assert out["dist"] == ("zeros" if dist else "u(-0.5,0.5)")
    assert out["steps"] == 3 and out["warmup"] == 1 and out["peak"] == 2500.0
    assert 0 < out["frac"] < 1 and abs(out["frac"] - out["achieved"] / out["peak"]) < 1e-4
    assert 0 < out["kernel_ms"]["min"] <= out["kernel_ms"]["median"]


def test_latency_floor_lists_its_launches():
    """bench.py --floor: one stderr line per launch it times, each with a positive device time
    per launch from graph replays; nothing on stdout."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--floor"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert not r.stdout.strip()
    lines = [json.loads(ln) for ln in r.stderr.splitlines() if ln.startswith('{"floor"')]
    assert len(lines) == 6, r.stderr[-2000:]
    assert all(d["graph_us_per_launch"] > 0 for d in lines)
    assert [(d.get("M"), d.get("N"), d.get("K")) for d in lines[1:]] == [
        (512, 512, 0), (32, 32, 64), (512, 512, 64), (512, 512, 512), (1024, 768, 128)]
