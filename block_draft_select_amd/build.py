"""Build libdflash.so in-tree with hipcc for gfx950.

Usage: ``python block_draft_select_amd/build.py`` (run by path: importing the
package needs the built library), or ``__graft_entry__.build()``.
Every source is compiled on each call; objects go to ``_build/`` next to this
file and the library to ``block_draft_select_amd/libdflash.so``.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdflash.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic stays off: the compiler must not form
    # v_pk_{add,mul,fma}_f32 from scalar float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: in the AGPR form the streaming
    # kernel's gate blocks added AGPRs on top of its VGPRs, and the total
    # sets every block's occupancy
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libdflash.so")


def _compile(src, obj, extra):
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False, save_temps=False):
    """Compile every HIP/C++ source of the library and link libdflash.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    extra = ["-save-temps=obj"] if save_temps else []
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for s in srcs:
            obj = os.path.join(BUILD_DIR, os.path.basename(s) + ".o")
            jobs.append(ex.submit(_compile, s, obj, extra))
        objs = [j.result() for j in jobs]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
