"""Host-side pieces of the offline tuner (dense_gemm_f16f32_amd/tune.py): the table it writes
is what the planner compiles in, so its format and keys are checked here without a GPU."""
import json
import math

import dense_gemm_f16f32_amd as g
from dense_gemm_f16f32_amd import tune
from test_abi import shape_class, tune_entries


def fake_results():
    rows = []
    for K in (64, 4096):
        for M in (32, 4096, 8192):
            for N in (32, 768, 8192):
                best = g.TILE_256x256x64 if min(M, N) >= 4096 else g.TILE_32x64x64
                big = best == g.TILE_256x256x64
                rows.append({"M": M, "N": N, "K": K, "best_tile": best,
                             "group_m": 4 if big and K == 4096 else (1 if big else 0),
                             "remap": 2 if big and K == 64 else 0,
                             "current": g.TILE_128x64x64,
                             "us": {str(best): 10.0, str(g.TILE_128x64x64): 12.5},
                             "ab_us": {}, "group_us": {"4": 9.5, "1x": 9.25},
                             "auto_us": 12.0})
    return rows


def test_written_rows_parse_back(tmp_path, monkeypatch):
    out = tmp_path / "table.inc"
    rows = fake_results()
    tune.write_table(str(out), rows, "test device", "0123456789abcdef")
    import test_abi
    monkeypatch.setattr(test_abi, "TUNE_TABLE", str(out))
    parsed = tune_entries()
    assert len(parsed) == len(rows)
    for r in rows:
        key = shape_class(r["M"], r["N"], r["K"])
        assert parsed[key] == (r["best_tile"], r["group_m"], r["remap"]), r
    text = out.read_text()
    assert "test device" in text and "12.5" in text       # the replaced choice's time
    assert "9.25" in text                                  # G = 1 with the permutation off


def test_keys_are_rounded_log2():
    # 768 = 2^9.58 rounds to class 10; the writer and the planner's lookup agree on it
    assert int(round(math.log2(768))) == 10 == shape_class(1, 768, 1)[1]
    assert shape_class(1, 1, 1) == (5, 5, 6) and shape_class(1 << 20, 1 << 20, 1 << 20) == (13, 13, 13)


def test_rewrite_from_json(tmp_path):
    rec = {"device": "d", "results": fake_results()}
    js = tmp_path / "sweep.json"
    js.write_text(json.dumps(rec))
    out = tmp_path / "t.inc"
    import sys
    argv = sys.argv
    try:
        sys.argv = ["tune", "--from-json", str(js), "--out", str(out)]
        tune.main()
    finally:
        sys.argv = argv
    assert out.read_text().count("\n{") == len(rec["results"])


def test_merge_partial_sweeps_with_the_source_hash(tmp_path):
    rows = fake_results()
    a, b = tmp_path / "a.json", tmp_path / "b.json"
    a.write_text(json.dumps({"device": "d", "source_hash": "00ff00ff00ff00ff",
                             "results": [r for r in rows if r["K"] == 64]}))
    b.write_text(json.dumps({"device": "d", "source_hash": "00ff00ff00ff00ff",
                             "results": [r for r in rows if r["K"] != 64]}))
    out = tmp_path / "t.inc"
    import sys
    argv = sys.argv
    try:
        sys.argv = ["tune", "--from-json", f"{a},{b}", "--out", str(out)]
        tune.main()
        text = out.read_text()
        assert text.count("\n{") == len(rows) and "kernel source hash 00ff00ff00ff00ff" in text
        b.write_text(json.dumps({"device": "d", "source_hash": "1111111111111111",
                                 "results": [r for r in rows if r["K"] != 64]}))
        sys.argv = ["tune", "--from-json", f"{a},{b}", "--out", str(out)]
        try:
            tune.main()
            raise AssertionError("sweeps of different kernel sources were merged")
        except SystemExit:
            pass
    finally:
        sys.argv = argv


def test_shipped_table_was_measured_on_the_shipped_kernels():
    """The dispatch table's header names the kernel source hash it was swept at; it must be
    the hash of the kernels that ship (re-run the sweep after changing them)."""
    import re
    from dense_gemm_f16f32_amd.build import kernel_source_hash
    text = open(tune.TABLE).read()
    m = re.search(r"kernel source hash ([0-9a-f]{16})", text)
    assert m, "the table names no kernel source hash"
    assert m.group(1) == kernel_source_hash()
