"""bench.py's accounting, on the CPU: the algorithmic bytes are the
minimum of every tensor touched once (per token per batch row (6 Hk Dk +
5 Hv Dv + 6 Hv) elements over both calls, plus the state checkpoints), the
useful work is 7 + 15 flops per state element per step, and a run asked for
more than one GPU exits before touching any device."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_token():
    B, T, Hk, Hv, Dk, Dv, esz = 1, 2048, 16, 64, 192, 128, 2
    for nch in (1, 32):
        fwd, bwd = bench.algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, nch)
        state = B * Hv * Dv * Dk * 4
        # forward: q, k, v, g, beta in, y out; the nch chunk-start states and
        # S_T out.  backward: q, k, v, g, beta, dy in and dq, dk, dv, dg, dbeta
        # out; the nch states in, dS0 out
        assert fwd == B * T * (2 * Hk * Dk + 2 * Hv * Dv + 2 * Hv) * esz + (nch + 1) * state
        assert bwd == B * T * (4 * Hk * Dk + 3 * Hv * Dv + 4 * Hv) * esz + (nch + 1) * state
        assert (fwd + bwd - 2 * (nch + 1) * state) == B * T * (6 * Hk * Dk + 5 * Hv * Dv
                                                              + 6 * Hv) * esz
    f0, b0 = bench.algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, 32)
    f1, b1 = bench.algorithmic_bytes(B, T, Hk, Hv, Dk, Dv, esz, 32, s0=True, dst=True)
    assert (f1 - f0, b1 - b0) == (B * Hv * Dv * Dk * 4,) * 2  # S0 in, dS_T in


def test_useful_flops():
    assert (bench.FLOPS_FWD, bench.FLOPS_BWD) == (7, 15)
    assert bench.FP32_PEAK_TF == 157.3 and bench.HBM_PEAK_GBS == 8000.0


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
