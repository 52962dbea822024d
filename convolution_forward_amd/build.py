"""Build libconvfwd.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m convolution_forward_amd.build

Each source compiles to an object under _build/ (in parallel), then hipcc
links the shared library into convolution_forward_amd/_lib/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libconvfwd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    # Never emit packed fp32 instructions (v_pk_add/mul/fma_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE subnormals for fp32 on the device.
    "-fno-gpu-flush-denormals-to-zero",
    "-I" + INCLUDE, "-I" + CSRC,
]

# Per-source extra flags. Depthwise files must never fuse a product with the
# following sum (exact mode); fast mode uses explicit fma calls.
EXTRA_FLAGS = {
    "depthwise_direct.hip": ["-ffp-contract=off"],
    "depthwise_tiled.hip": ["-ffp-contract=off"],
    "depthwise_pad.hip": ["-ffp-contract=off"],
    "depthwise_planes.hip": ["-ffp-contract=off"],
    "depthwise_rows.hip": ["-ffp-contract=off"],
}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _up_to_date(src: str, obj: str) -> bool:
    """Object newer than its source and every header it may include."""
    if not os.path.exists(obj):
        return False
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps += [os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE)]
    deps.append(os.path.abspath(__file__))
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(d) < t for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    if incremental and _up_to_date(src, obj):
        return obj
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (only changed ones with incremental=True) and link."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
