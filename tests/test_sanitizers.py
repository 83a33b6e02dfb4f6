"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU).

* The C oracle with a driver that gives every tensor its own exactly sized heap
  block (tests/sanitize/oracle_asan.c).
* The C-ABI layer's validation and planning (ssm_abi.cpp, s6_plan.cpp,
  s6_bwd_plan.cpp), built host-only, with kernel launches replaced by
  stand-ins that abort, driven by a fuzzer over edge and random sizes
  (tests/sanitize/abi_fuzz.cpp).  Every
  fuzzed call must be refused before it could reach the HIP runtime, and the
  size arithmetic must not overflow.

Device code is not built: the sanitizers apply to host code only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_21_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", os.path.join(ROOT, "oracle", "ssm_oracle.c"),
          os.path.join(HERE, "oracle_asan.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "no finding" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm compilers")
def test_abi_validation_under_sanitizers(tmp_path):
    # host-side compile only: each sanitizer flag is given to the host pass
    flags = ["--offload-host-only", "-O1", "-g", "-std=c++17",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-x", "hip"]
    objs = []
    for src in (os.path.join(CSRC, "ssm_abi.cpp"), os.path.join(CSRC, "s6_plan.cpp"),
                os.path.join(CSRC, "s6_bwd_plan.cpp"),
                os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_fuzz.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_fuzz")
    _run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe])
    env = dict(ENV)
    for k in ("SSM_S6_SEGMENTS", "SSM_S6_LANES"):
        env.pop(k, None)
    r = _run([exe, "300000"], env=env)
    assert "no finding" in r.stdout
    env["SSM_S6_SEGMENTS"] = "7"                 # the planner's override path
    r = _run([exe, "50000"], env=env)
    assert "no finding" in r.stdout
