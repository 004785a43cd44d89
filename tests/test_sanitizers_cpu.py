"""Host-only AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU, no GPU).

* The CPU oracle (oracle/tg_oracle.c) with a driver that calls every function
  on small problems at the edges of their arguments and on refused ones
  (tests/sanitize/oracle_checks.c); leaks are reported too.
* The C ABI's host side (tiled_dense_gemm_09_amd/csrc/tg_api.cpp, host code
  instrumented) with a driver that feeds it invalid, overflowing and
  degenerate arguments and sweeps the host helpers
  (tests/sanitize/abi_checks.cpp); the kernel files' launchers are replaced
  by stubs that abort, so any call that would launch fails the check.

Both stop at the first report (no recovery)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="3")


def run_checked(exe, env):
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, "%s failed (%d):\n%s\n%s" % (exe, r.returncode, r.stdout[-2000:],
                                                          r.stderr[-6000:])
    assert "runtime error" not in r.stderr, r.stderr[-6000:]
    return r.stdout


def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    subprocess.check_call([
        gcc, "-std=c11", "-D_DEFAULT_SOURCE", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
        "-o", exe, os.path.join(ROOT, "oracle", "tg_oracle.c"),
        os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-lm"])
    assert "oracle checks passed" in run_checked(exe, SAN_ENV)


def test_abi_host_validation_under_address_and_undefined_behaviour_sanitizers():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm compilers not found")
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "tiled_dense_gemm_09_amd", "csrc")
    # the sanitizers instrument the host code only (the device code of
    # tg_api.cpp is compiled as usual and never runs here)
    host_san = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    common = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17",
              "-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), "-I", csrc] + host_san
    objs = []
    for src in (os.path.join(csrc, "tg_api.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run(common + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exe = os.path.join(OUT, "abi_checks")
    subprocess.check_call([clangxx, "-fsanitize=address,undefined", "-o", exe] + objs +
                          ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    # the HIP runtime's own allocations at exit are not this code's: leak
    # detection off for this one
    env = dict(SAN_ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0")
    assert "abi host checks passed" in run_checked(exe, env)
