"""Build the gfx950 HIP library ``libloom.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only (``--offload-arch=gfx950``)
with packed-FP32 instruction selection disabled, then linked into one shared
library next to this file.  Objects go to ``_build/`` (not tracked).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libloom.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 8, out: str = OUT, defines=()) -> str:
    """Compile and link; always rebuilds (the build check must compile).

    ``defines`` (e.g. ``["LOOM_ROW_SUMS_DEPTH=12"]``) override the kernels'
    schedule constants for a tuning build written to ``out``."""
    build_dir = BUILD if out == OUT else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), sources()))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
