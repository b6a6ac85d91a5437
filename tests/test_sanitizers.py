"""Host sanitizer runs (CPU only, no GPU).

* The fp64 oracle (oracle/based_oracle.c) built with AddressSanitizer and
  UndefinedBehaviorSanitizer (gcc), with the oracle's pin tests run against
  that build: a memory or UB error anywhere in the recurrence, the JRT prefix,
  the decode step or their threading fails the run.
* The C-ABI layer (csrc/capi.hip) compiled for the host only with the same
  sanitizers, linked against stub launchers, driven through every entry point
  by tests/sanitize/capi_driver.hip (validation, aliasing checks, dispatch).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "based_oracle.c")
# sanitizers for host code only (the C-ABI layer has no device code in this build)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", *GCC_SAN, "-fPIC", "-shared", "-std=c99", "-o", str(so),
                           ORACLE_SRC, "-lm", "-lpthread"])
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", BLA_ORACLE_LIBRARY=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py", "tests/test_oracle_compact.py",
                        "tests/test_oracle_padding.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out


def test_capi_layer_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not installed")
    inc = os.path.join(ROOT, "include")
    objs = []
    for src in (os.path.join(ROOT, "recurrent_lm_sequence_amd", "csrc", "capi.hip"),
                os.path.join(ROOT, "tests", "sanitize", "capi_driver.hip")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.check_call([hipcc, "--offload-host-only", "-O1", "-g", "-std=c++17", *HOST_SAN,
                               "-I", inc, "-c", src, "-o", str(obj)])
        objs.append(str(obj))
    exe = tmp_path / "capi_driver"
    subprocess.check_call([clang, *GCC_SAN, *objs, "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
                                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations hold" in r.stdout
