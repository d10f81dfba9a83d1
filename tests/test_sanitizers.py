"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (``oracle/rat_oracle.c``) with gcc, driven by
  ``tests/sanitize/oracle_driver.c`` through every entry point on a tiny case
  (leak checking on).
* The library's host code (``csrc/*.hip`` with the sanitizers on the host
  pass only; device code is built as usual), linked into
  ``tests/sanitize/abi_driver.cpp``, which calls the pure host helpers and the
  validation of every entry point.  Nothing is launched, so no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...: rc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp", "-std=c11", "-Wall",
          "-Wno-unknown-pragmas", os.path.join(ROOT, "oracle", "rat_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    assert "oracle driver: ok" in _run([exe], env=env)


def test_host_abi_under_asan_ubsan():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    from dilated_sparse_attention_rat_amd import build as b
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in b.sources():
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        # sanitizers on the host pass only: -Xarch_host before each option
        _run([hipcc, *b.HIPCC_FLAGS, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
              "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
              "-c", src, "-o", obj])
        objs.append(obj)
    drv = os.path.join(OUT, "abi_driver.o")
    _run([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = os.path.join(OUT, "abi_driver")
    _run([clangxx, "-fsanitize=address,undefined", drv, *objs, "-o", exe,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    # the HIP runtime keeps allocations until exit: leak checking off here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    assert "abi driver: ok" in _run([exe], env=env)
