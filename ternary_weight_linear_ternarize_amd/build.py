"""Build libbitlinear.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m ternary_weight_linear_ternarize_amd.build

Every source is compiled with hipcc for --offload-arch=gfx950 and the numeric
flags the kernels rely on: no floating-point contraction, correctly rounded
binary32 divide and sqrt, and the packed-fp32 feature switched off.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbitlinear.so")

SOURCES = ["api.hip", "pack.hip", "quant.hip", "gemv.hip", "gemm.hip", "bin1.hip", "a48.hip", "skinny.hip", "ksplit.hip", "probe.hip"]
HEADERS = ["bl_device.h", "bl_launch.h", "gemm_tiles.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature: harmless warning
    noise = [l for l in r.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    return obj, "\n".join(noise)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, msg in results:
        if verbose and msg:
            print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *[o for o, _ in results], "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
