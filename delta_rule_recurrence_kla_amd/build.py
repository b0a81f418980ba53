"""Build libkla.so (HIP kernels + C ABI) for gfx950, in tree.

    python -m delta_rule_recurrence_kla_amd.build [-v]

Objects go to _build/ at the repository root; the library goes to
delta_rule_recurrence_kla_amd/lib/libkla.so. Every HIP source is compiled with
packed fp32 instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
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
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libkla.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kla_prep.hip", "kla_state.hip", "kla_state_dma.hip", "kla_decode.hip", "kla_loglinear.hip", "kla_bwd.hip",
           "kla_scratch.hip", "kla_api.cpp"]
# MFMA results go to ordinary VGPRs (-amdgpu-mfma-vgpr-form) rather than accumulation
# registers: every accumulator here is read back by vector instructions (splits, scalings,
# stores), and with the accumulation-register form each such read costs a v_accvgpr_read
# (about 125 of them per chunk in the state kernel, 3% of its time).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wall"]
# The prep kernel is a latency-bound chain of MFMA, LDS and VALU work at two waves per SIMD;
# LLVM's iterative ILP scheduler orders it better than the default occupancy scheduler
# (about 5% on gfx950). The DMA state kernel keeps the default scheduler: with its copy wave
# it has a 256-register budget, under which the ILP scheduler's output fails register
# allocation in this compiler, and with MFMA results in VGPRs the default one was already
# the faster of the two for it.
PER_FILE = {
    "kla_prep.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
