"""The CPU-side native code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two libraries run on the host: the oracle (plain C) and the library's host
core (the C ABI's checks, state machine and launch plan), which CPU tests
link against a recording backend.  This test builds both with
-fsanitize=address,undefined (errors fatal), preloads the sanitizer
runtimes into a child Python, points the loaders at the sanitized builds
(AFD_ORACLE_LIB, AFD_HOSTFAKE_LIB) and runs their CPU test files there: any
out-of-bounds access, use after free or undefined behaviour in them aborts
the child and fails this test.  Only gcc/g++ are used (the GPU library is
not part of it)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

# CPU test files whose native calls go through the two libraries
FILES = ["tests/test_host_core.py", "tests/test_oracle_config.py", "tests/test_oracle_layout.py",
         "tests/test_oracle_combine.py", "tests/test_oracle_staged.py", "tests/test_golden.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_native_cpu_code_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    oracle_lib = str(tmp_path / "liboracle_san.so")
    fake_lib = str(tmp_path / "libafd_hostfake_san.so")
    subprocess.check_call(["gcc", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas",
                           *SAN, os.path.join(ROOT, "oracle", "afd_oracle.c"), "-o", oracle_lib, "-lm"])
    csrc = os.path.join(ROOT, "combine_layout_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", *SAN,
                           f"-I{os.path.join(ROOT, 'include')}", os.path.join(csrc, "afd_core.cpp"),
                           os.path.join(csrc, "afd_backend_fake.cpp"), "-o", fake_lib])
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{asan}:{ubsan}",
        # the Python interpreter and torch are not built with the sanitizers:
        # leaks at exit and their own allocator pairings are not checked
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "AFD_ORACLE_LIB": oracle_lib,
        "AFD_HOSTFAKE_LIB": fake_lib,
    })
    # the symbol-export check loads the GPU library, which is not built with
    # the sanitizers; the large workloads run the same code paths as the
    # small cases on arrays whose shadow memory makes them slow here
    skip = ["exports_every_declared_symbol", "3a1f", "fp8_prefill", "1a3f", "skew_h4096", "config_pins_all",
            "combine_of_partials[2", "masked_single_rounding_combine[0", "masked_single_rounding_combine[2"]
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                           "-k", " and ".join(f"not {k}" for k in skip), *FILES],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (proc.stdout[-3000:] + proc.stderr[-3000:])
    assert proc.returncode == 0, tail
    assert " passed" in proc.stdout, tail
