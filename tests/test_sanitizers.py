"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

gdr_api.hip (argument checks, size arithmetic, the per-device scratch lookup
table, the launch set-up) is compiled with the sanitizers on its host pass
only, linked with the kernel objects of the regular build and driven by
tests/abi_host_check.c, which calls every size query over a spread of shapes
and checkpoint intervals and every argument-rejection path.  No call reaches
the device, so this runs without a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_recurrence_amd", "csrc")
BUILD = os.path.join(CSRC, "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_host_code_under_asan_ubsan(tmp_path):
    from gated_delta_rule_recurrence_amd import build
    objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))] if os.path.isdir(BUILD) else []
    if not any(o.endswith("gdr_chunk.o") for o in objs):
        build.build(verbose=False)
        objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))]
    kernel_objs = [o for o in objs if o.endswith(".o") and not o.endswith("gdr_api.o")]
    inc = os.path.join(ROOT, "include")
    api = tmp_path / "gdr_api_san.o"
    drv = tmp_path / "abi_host_check.o"
    exe = tmp_path / "abi_host_check"
    run = lambda cmd: subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    # sanitizers on the host pass only (the device code is built as usual)
    r = run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{inc}", "-c", os.path.join(CSRC, "gdr_api.hip"), "-o", str(api)])
    assert r.returncode == 0, r.stderr
    r = run([CLANG, "-g", "-O1", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", f"-I{inc}", "-c",
             os.path.join(ROOT, "tests", "abi_host_check.c"), "-o", str(drv)])
    assert r.returncode == 0, r.stderr
    r = run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", str(drv), str(api), *kernel_objs,
             "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "abi host checks passed" in out
