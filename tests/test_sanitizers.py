"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The library: every source of libkla compiled as the library build does (gfx950 device
  code) with ASan and UBSan on the host pass only, linked with
  tests/sanitize/abi_checks.cpp, which drives every
  entry point through its validation, the planner over a grid of sizes, the alignment
  rule, the no-allocation entry point's size limit and the timing hook. No check reaches
  a kernel launch (there is no GPU here, and validation settles each call first).
* The C oracle (oracle/kla_ref.c), compiled with gcc under both sanitizers and driven by
  tests/sanitize/oracle_checks.c: forwards over all heads and head lists, ragged sizes,
  both write-strength modes, zero keys with eps = 0, decode steps and bad arguments.

Any sanitizer report fails the test (UBSan is built not to recover).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "delta_rule_recurrence_kla_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{msg[-4000:]}"
    return r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain absent")
def test_library_host_code_under_asan_ubsan(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp"))
    srcs = [os.path.join(CSRC, f) for f in srcs] + [os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")]
    def compile_one(s):
        o = os.path.join(tmp_path, os.path.basename(s) + ".o")
        # each sanitizer flag applies to the host compilation alone (-Xarch_host)
        _run([HIPCC, "-x", "hip", f"--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined", "-c", s, "-o", o])
        return o

    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(tmp_path, "abi_checks")
    _run([CLANG, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = _run([exe], env=SAN_ENV, timeout=300)
    assert "abi checks passed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc absent")
def test_c_oracle_under_asan_ubsan(tmp_path):
    exe = os.path.join(tmp_path, "oracle_checks")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "kla_ref.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-lm", "-o", exe])
    out = _run([exe], env=SAN_ENV, timeout=300)
    assert "oracle checks passed" in out
