"""Build the gfx950 attention library in-tree: csrc/*.hip -> libattn_fa2.so.

Usage: python -m attention_fa2_fwd_amd.build   (or build() from Python).
Each translation unit is compiled by hipcc for gfx950 only, in parallel, and
linked into one shared library next to this file.  Packed-fp32 VALU
instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libattn_fa2.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


# Per-source extra flags.  The forward kernel never produces or consumes NaN
# (masked scores are -inf, which stays honoured), so max/min need no
# NaN-quieting of their inputs.
EXTRA_FLAGS = {"fwd_bf16.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, cc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = EXTRA_FLAGS.get(os.path.basename(src), [])
    cmd = [cc, *DEVICE_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line)    # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every kernel source for gfx950 and link libattn_fa2.so."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 8))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build()
