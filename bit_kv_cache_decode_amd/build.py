"""Build libkivi.so in-tree for gfx950 with hipcc.

Usage: ``python -m bit_kv_cache_decode_amd.build`` (or ``build()``).  Always
recompiles.  The HIP source is built with packed-fp32 instructions disabled;
the host-only C ABI source is built by hipcc as plain C++.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkivi.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every atomic in the library is issued by one lane; the atomic optimizer
    # would turn it into a per-wave atomic whose result is read back at once,
    # stalling the wave on a device-scope round trip where the result is
    # only needed at the end of the kernel
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + res.stdout)
    return res.stdout


def build(verbose=False, save_temps=False):
    os.makedirs(BUILD, exist_ok=True)
    k_obj = os.path.join(BUILD, "kivi_kernels.o")
    a_obj = os.path.join(BUILD, "kivi_api.o")
    extra = ["-save-temps=obj"] if save_temps else []
    log = _run([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, "kivi_kernels.hip"), "-o", k_obj])
    log += _run([HIPCC, *CXX_FLAGS, "-x", "c++", "-c", os.path.join(CSRC, "kivi_api.cpp"), "-o", a_obj])
    tmp = OUT + ".tmp"
    log += _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", k_obj, a_obj, "-o", tmp])
    os.replace(tmp, OUT)
    if verbose:
        print(log)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
