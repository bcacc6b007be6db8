"""Ahead-of-time build of the native libraries (no JIT).

  _lib/libafd.so           the library: host core + gfx950 kernels (hipcc)
  _lib/libafd_hostfake.so  the host core over a recording backend (g++), used
                           only by CPU tests of the state machine and checks
  _lib/libafd_clock.so     device clock stamps for the benchmark's timing
                           inside captured graphs (hipcc)
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libafd.so")
FAKE_LIB = os.path.join(LIBDIR, "libafd_hostfake.so")
CLOCK_LIB = os.path.join(LIBDIR, "libafd_clock.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # no packed-FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel-argument preloading: a kernel's leading scalar arguments (up to
    # nine, as many as the user SGPRs hold) arrive in SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=9",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    subprocess.check_call(cmd)


def build_lib(extra=()):
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, *HIP_FLAGS, *extra, os.path.join(CSRC, "afd_core.cpp"),
          os.path.join(CSRC, "afd_kernels.hip"), "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_fake():
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = FAKE_LIB + ".tmp%d" % os.getpid()
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
          f"-I{os.path.join(ROOT, 'include')}",
          os.path.join(CSRC, "afd_core.cpp"), os.path.join(CSRC, "afd_backend_fake.cpp"), "-o", tmp])
    os.replace(tmp, FAKE_LIB)
    return FAKE_LIB


def build_clock():
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = CLOCK_LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, *HIP_FLAGS, os.path.join(CSRC, "afd_clock.hip"), "-o", tmp])
    os.replace(tmp, CLOCK_LIB)
    return CLOCK_LIB


def build_all():
    build_fake()
    build_lib()
    build_clock()


if __name__ == "__main__":
    build_all()
    print(LIB)
    print(FAKE_LIB)
    print(CLOCK_LIB)
