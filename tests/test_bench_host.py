"""Host-side behaviour of bench.py that needs no GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_record_matches_current_kernel_and_plan():
    """The committed record is for the launch configuration the planner picks at 8192^3 and
    was taken with the kernels that ship."""
    import dense_gemm_f16f32_amd as g
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    rc, p = g.gemm_f16f32_plan(8192, 8192, 8192, 1 << 40, 2 << 40, 3 << 40, 8192, 8192, 8192)
    assert rc == g.OK
    key = f"gemm8192_u/tile{p['tile']}/g{p['group_m']}/remap{p['xcd_remap']}"
    e = rec[key]
    fetch = e["fetch_size_kib_per_dispatch"] * 1024 * e["fetch_factor"]
    write = e["write_size_kib_per_dispatch"] * 1024 * e["write_factor"]
    assert abs(fetch + write - e["bytes_per_launch"]) < 1e3
    assert e["algorithmic_bytes_per_launch"] == 2 * 3 * 8192 * 8192
    assert e["source_hash"] == bench.kernel_source_hash()
    assert bench.measured_traffic("gemm8192_u", p["tile"], p["group_m"], p["xcd_remap"]) == \
        e["bytes_per_launch"]
    # any other launch configuration reports no traffic
    assert bench.measured_traffic("gemm8192_u", p["tile"], p["group_m"] + 1,
                                  p["xcd_remap"]) is None
    assert bench.measured_traffic("gemm4096_u", p["tile"], p["group_m"], p["xcd_remap"]) is None


def test_traffic_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    rec = {"w/tile1/g8/remap1": {"source_hash": "0000", "bytes_per_launch": 5}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic("w", 1, 8, 1) is None
    rec["w/tile1/g8/remap1"]["source_hash"] = bench.kernel_source_hash()
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("w", 1, 8, 1) == 5


def test_source_hash_ignores_comments():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    assert bench.strip_comments(code) == bench.strip_comments(
        "int f(int x) { return x + 1; }")
    assert bench.strip_comments(code) != bench.strip_comments("int f(int x) { return x + 2; }")


def test_smi_parser():
    # the layout `amd-smi metric -c -p` prints (ROCm 7): a POWER block, then one block per
    # clock domain; only the GFX_<n> clocks and the socket power are taken
    text = """GPU: 0
    POWER:
        SOCKET_POWER: 1399 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1745 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1762 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 2000 MHz
        VCLK_0:
            CLK: 29 MHz
"""
    assert bench.parse_smi(text) == ([1745, 1762], 1399.0)
    assert bench.parse_smi("") == ([], None)
