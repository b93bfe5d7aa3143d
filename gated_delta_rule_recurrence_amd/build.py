"""Build libgdr.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m gated_delta_rule_recurrence_amd.build [--jobs N]

Every .hip file under csrc/ is compiled to an object in csrc/_build/ and the
objects are linked into gated_delta_rule_recurrence_amd/libgdr.so.  Packed
FP32 instructions are disabled for all device code
(-target-feature -packed-fp32-ops); hipcc's host pass prints a harmless
warning that it does not know that feature.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = CSRC / "_build"
LIB = PKG / "libgdr.so"
INCLUDE = PKG.parent / "include"
# test-only probes of the device helpers (not part of libgdr.so)
PROBE_SRC = PKG.parent / "tests" / "probe" / "gdr_device_probe.hip"
PROBE_LIB = PROBE_SRC.parent / "libgdr_probe.so"

ARCH = "gfx950"
CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unknown-warning-option",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libgdr)")
    return exe


def _compile(src: Path) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *CXXFLAGS, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{res.stdout}\n{res.stderr}")
    # keep real diagnostics, drop the known host-pass feature notice
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stderr or "").splitlines() if noise not in ln]
    if any(m.strip() for m in msgs):
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> Path:
    """Compile every HIP source and link libgdr.so; returns its path."""
    BUILD.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    if not sources:
        raise RuntimeError(f"no .hip sources in {CSRC}")
    # objects of sources that no longer exist (the sanitizer test links
    # every object in the build folder)
    stems = {src.stem for src in sources}
    for obj in BUILD.glob("*.o"):
        if obj.stem not in stems:
            obj.unlink()
    jobs = jobs or min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if PROBE_SRC.exists():
        build_probe()
    if verbose:
        print(f"built {LIB} from {len(sources)} sources")
    return LIB


def build_probe() -> Path:
    """The test-only probe library of the device helpers."""
    tmp = PROBE_LIB.with_name(PROBE_LIB.name + ".tmp")
    cmd = [hipcc(), *CXXFLAGS, "-shared", str(PROBE_SRC), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC.name}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs)


if __name__ == "__main__":
    main()
