"""The boundary itself: the C-ABI from a plain C program, and calls from several host threads.

* tests/c_abi_check (C99, built by __graft_entry__.build() from tests/c_abi_check.c) allocates
  with the HIP runtime and calls gemm_f16f32, gemm_f16f32_strided (column-major C) and
  gemm_f16f32_strided_ws (split K) -- no Python, no torch in that process.  Its results must
  meet the oracle's bar and equal the same calls made through the Python binding, bit for bit.
* The library keeps no state, so host threads may call it at the same time on their own
  streams: four threads, each with its own stream and problems (split K with its own
  workspace among them), must reproduce the single-threaded results bit for bit.
"""
import os
import subprocess
import threading

import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import assert_within_tolerance, from_dev, to_dev
from synthetic_inputs import operands

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi_check")

torch = pytest.importorskip("torch")


def test_c_program_is_built():
    """(CPU) the plain-C check exists, loads its libraries and checks its arguments."""
    assert os.path.exists(EXE), "tests/c_abi_check is missing: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(300, 264, 1000), (129, 65, 4093)])
def test_c_program_uses_the_abi(tmp_path, M, N, K):
    A, B = operands(M, N, K, "u(-0.5,0.5)", M + N + K)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(A.tobytes())
        f.write(B.tobytes())
    print(f"c_abi_check {M} {N} {K}", flush=True)
    r = subprocess.run([EXE, str(M), str(N), str(K), str(src), str(dst)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("done")
    out = np.fromfile(dst, dtype=np.uint16).reshape(3, M, N)
    want = oracle.gemm(A, B)
    for i, what in enumerate(("gemm_f16f32", "strided, column-major C", "split K = 4")):
        assert_within_tolerance(out[i], want, f"C program: {what}")
    Ad, Bd = to_dev(A), to_dev(B)
    assert np.array_equal(out[0], from_dev(g.matmul(Ad, Bd)))
    assert np.array_equal(out[1], out[0])
    assert np.array_equal(out[2], from_dev(g.matmul(Ad, Bd, split_k=4)))


@pytest.mark.gpu
def test_concurrent_host_threads_on_their_own_streams():
    problems = [(700, 500, 900, {}), (256, 256, 8192, {"split_k": 8}), (1000, 1000, 300, {}),
                (64, 4096, 2048, {"split_k": g.SPLIT_K_AUTO}), (513, 257, 1025, {"tile": 9}),
                (300, 300, 3000, {"split_k": 3}), (2048, 128, 700, {}), (1, 1000, 5000, {})]
    dev = []
    for i, (M, N, K, opts) in enumerate(problems):
        A, B = operands(M, N, K, "n(0,0.1)", 100 + i)
        dev.append((to_dev(A), to_dev(B), opts))
    want = [from_dev(g.matmul(Ad, Bd, **opts)) for Ad, Bd, opts in dev]
    for w, (M, N, K, _) in zip(want, problems):
        assert w.shape == (M, N)
    torch.cuda.synchronize()
    errors, results = [], {}

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rep in range(4):
                    for j in range(t, len(dev), 4):
                        Ad, Bd, opts = dev[j]
                        results[(t, rep, j)] = g.matmul(Ad, Bd, **opts)
            s.synchronize()
        except Exception as e:  # noqa: BLE001 -- reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    assert len(results) == 4 * len(dev)
    for (t, rep, j), C in results.items():
        assert np.array_equal(from_dev(C), want[j]), (t, rep, j)
