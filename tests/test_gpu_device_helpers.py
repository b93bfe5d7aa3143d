"""The device helpers of gdr_device.h on the GPU, bit for bit against CPU
models (in-bounds probe kernels in tests/probe, a test-only library):

* split3_quad, the exact three-piece bf16 split every bf16-product kernel
  uses: the same pieces as the numpy model of tests/test_kernel_math.py
  (fp32 remainders, each piece rounded to nearest even), over random values
  from 2^-100 to 2^100 and random bit patterns below bf16 overflow;
* lds_read_tr16 (ds_read_b64_tr_b16): inside each group of 16 lanes, lane i
  receives element i % 4 of the 8-byte blocks named by lanes i / 4,
  4 + i / 4, 8 + i / 4 and 12 + i / 4, in that order;
* tile_operand: from a swizzled row-major bf16 tile, lane l gathers rows
  k0 + 8 (l / 16) + 0..7 of column n0 + l % 16, element e in bits 16e...;
* the compute-peak loops that bench.py times count exactly.
"""
import ctypes
import os

import numpy as np
import pytest

from test_kernel_math import _wide_fp32, split3

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libgdr_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        from gated_delta_rule_recurrence_amd import build
        build.build_probe()
    lib = ctypes.CDLL(PROBE)
    vp = ctypes.c_void_p
    lib.gdr_probe_split3.argtypes = [vp, vp, ctypes.c_int, vp]
    lib.gdr_probe_tr16.argtypes = [vp, vp, vp]
    lib.gdr_probe_tile_operand.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.gdr_probe_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    return lib


def test_split3_matches_cpu_model(cuda, probe):
    import torch
    x = _wide_fp32(np.random.default_rng(11), 1 << 19)
    x = np.concatenate([x, np.random.default_rng(12).standard_normal(1 << 19).astype(np.float32),
                        np.array([0.0, 1.0, -1.0, 0.5], np.float32)])
    n4 = x.size // 4
    xd = torch.from_numpy(x).to(cuda)
    out = torch.zeros(3 * n4 * 2, dtype=torch.int32, device=cuda)
    assert probe.gdr_probe_split3(xd.data_ptr(), out.data_ptr(), n4, None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(3, -1)
    for plane, ref in zip(got, split3(x)):
        want = (ref.view(np.uint32) >> 16).astype(np.uint16)
        np.testing.assert_array_equal(plane, want)


def test_tr16_lane_order(cuda, probe):
    import torch
    rng = np.random.default_rng(13)
    blk = rng.permutation(256)[:64].astype(np.int32)  # distinct blocks, in range
    bd = torch.from_numpy(blk).to(cuda)
    out = torch.zeros(256, dtype=torch.int16, device=cuda)
    assert probe.gdr_probe_tr16(bd.data_ptr(), out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4)
    lds = (np.arange(1024) ^ 0x5A5A).astype(np.uint16)
    want = np.zeros((64, 4), np.uint16)
    for lane in range(64):
        g, i = lane // 16, lane % 16
        for e in range(4):
            src = 16 * g + 4 * e + i // 4
            want[lane, e] = lds[4 * blk[src] + i % 4]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("k0", [0, 32])
@pytest.mark.parametrize("n0", [0, 16, 96, 176])
def test_tile_operand_gathers_columns(cuda, probe, k0, n0):
    import torch
    out = torch.zeros(512, dtype=torch.int16, device=cuda)
    assert probe.gdr_probe_tile_operand(k0, n0, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(64, 8)
    want = np.zeros((64, 8), np.uint16)
    for lane in range(64):
        for e in range(8):
            r, c = k0 + 8 * (lane // 16) + e, n0 + lane % 16
            want[lane, e] = (r * 192 + c) ^ 0x3C3C
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("kind,per_iter", [(0, None), (1, 512.0), (2, 64.0)])
def test_peak_loops_count_exactly(cuda, probe, kind, per_iter):
    """The compute-peak loops the benchmark times do the work they claim:
    the FMA chains a <- a/2 + 1 from a = 0..7 all reach 2 (sum 16); each
    bf16 MFMA of ones adds 32 to each of a wave's 4 x 4 accumulator values
    per lane (512 per iteration), each fp32 16x16x4 MFMA adds 4 (64)."""
    import torch
    iters, blocks = 3, 8
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device=cuda)
    assert probe.gdr_probe_peak(kind, blocks, iters, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    want = 16.0 if per_iter is None else per_iter * iters
    np.testing.assert_array_equal(out.cpu().numpy(), np.full(blocks * 256, want, np.float32))


def test_probe_rejects_bad_arguments(probe):
    """Host-side checks (no launch)."""
    assert probe.gdr_probe_tile_operand(5, 0, 16, None) == -1
    assert probe.gdr_probe_tile_operand(0, 184, 16, None) == -1
    assert probe.gdr_probe_split3(None, None, 4, None) == -1
    assert probe.gdr_probe_peak(3, 8, 1, 16, None) == -1
    assert probe.gdr_probe_peak(0, 0, 1, 16, None) == -1
    assert probe.gdr_probe_peak(0, 8, 0, 16, None) == -1
    assert probe.gdr_probe_peak(0, 8, 1, None, None) == -1
