"""ctypes view of include/afd.h (argument marshalling only).

The library is built ahead of time (``combine_layout_amd/build.py``) into
``combine_layout_amd/_lib/libafd.so``.  Loading fails loudly when it is
missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libafd.so")
# the host core over the recording backend, for CPU tests; AFD_HOSTFAKE_LIB
# points them at another build (the sanitizer test's)
FAKE_LIB_PATH = os.environ.get("AFD_HOSTFAKE_LIB") or os.path.join(HERE, "_lib", "libafd_hostfake.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "afd.h")

AFD_OK, AFD_E_ARG, AFD_E_SHAPE, AFD_E_ORDER, AFD_E_CAPACITY, AFD_E_ROUTE, AFD_E_HIP, AFD_E_TIMEOUT = \
    0, -1, -2, -3, -4, -5, -6, -7
AFD_BF16, AFD_FP8_E4M3 = 0, 1
AFD_COMBINE_ONCE, AFD_COMBINE_PER_STAGE, AFD_COMBINE_PER_STAGE_FP8 = 0, 1, 2
COMBINE_MODES = {"once": AFD_COMBINE_ONCE, "per_stage": AFD_COMBINE_PER_STAGE,
                 "per_stage_fp8": AFD_COMBINE_PER_STAGE_FP8}
AFD_DISPATCH_AUTO, AFD_DISPATCH_SPLIT, AFD_DISPATCH_ONE_LAUNCH = 0, 1, 2
DISPATCH_MODES = {"auto": AFD_DISPATCH_AUTO, "split": AFD_DISPATCH_SPLIT, "one_launch": AFD_DISPATCH_ONE_LAUNCH}
ROUTE_NONE, ROUTE_RANGE, ROUTE_NEG, ROUTE_DUP = 0, 1, 2, 3
MAX_SOURCES, MAX_PARTITIONS, MAX_EXPERTS, MAX_TOPK = 16, 16, 512, 32
STATIC_SCRATCH_BYTES = 64 << 20

STATUS_NAMES = {0: "AFD_OK", -1: "AFD_E_ARG", -2: "AFD_E_SHAPE", -3: "AFD_E_ORDER",
                -4: "AFD_E_CAPACITY", -5: "AFD_E_ROUTE", -6: "AFD_E_HIP", -7: "AFD_E_TIMEOUT"}


class Config(ctypes.Structure):
    _fields_ = [("num_sources", ctypes.c_int32), ("num_partitions", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("topk", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("expert_alignment", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("combine", ctypes.c_int32), ("dispatch", ctypes.c_int32)]


class Receipt(ctypes.Structure):
    _fields_ = [("round", ctypes.c_uint64), ("partition", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Receive(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("weights", ctypes.c_void_p),
                ("ends", ctypes.c_void_p), ("receive_rows", ctypes.c_int64), ("receipt", Receipt)]


class RoundInfo(ctypes.Structure):
    _fields_ = [("round", ctypes.c_uint64), ("dispatch_path", ctypes.c_int32),
                ("dispatch_kernels", ctypes.c_int32), ("combine_kernels", ctypes.c_int32),
                ("tokens", ctypes.c_int32), ("layout_tiles", ctypes.c_int32), ("tile_tokens", ctypes.c_int32)]


DISPATCH_PATHS = {0: "none", 1: "one_kernel", 2: "tiled", 3: "cached", 4: "empty", 5: "one_launch"}


class AfdError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

SIGNATURES = {
    "afd_query": ([ctypes.POINTER(Config), _I32, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_I64)], _I32),
    "afd_create": ([ctypes.POINTER(Config), _P, ctypes.c_size_t, ctypes.POINTER(_P)], _I32),
    "afd_create_static": ([ctypes.POINTER(Config), ctypes.POINTER(_P)], _I32),
    "afd_bind_partition": ([_P, _I32, _P, _P, _P, _I64], _I32),
    "afd_destroy": ([_P], _I32),
    "afd_source_dispatch": ([_P, _I32, _I32, _P, _P, _P, _P, _I64, _I64, _P, _I32, _I32, _P], _I32),
    "afd_source_dispatch_cached": ([_P, _I32, _I32, _P, _P, _P, _I64, _I64, _P, _I32, _P], _I32),
    "afd_worker_receive": ([_P, _I32, _I32, _I32, _P, ctypes.POINTER(Receive), _P], _I32),
    "afd_worker_reply": ([_P, _I32, _P, _I64, ctypes.POINTER(Receipt), _P], _I32),
    "afd_source_collect": ([_P, _I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_I64), _P], _I32),
    "afd_get_error": ([_P, _P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                       ctypes.POINTER(_I32)], _I32),
    "afd_get_partials": ([_P, _I32, _I32, ctypes.POINTER(_P), ctypes.POINTER(_I64)], _I32),
    "afd_get_round_info": ([_P, ctypes.POINTER(RoundInfo)], _I32),
    "afd_set_dispatch_wait": ([_P, _I32], _I32),
    "afd_status_string": ([_I32], ctypes.c_char_p),
}


def header_symbols():
    """Function names declared in include/afd.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:afd_status|const char \*)\s*(afd_\w+)\s*\(", text, re.M)))


def _bind(lib):
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = None


def load():
    """The HIP library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with combine_layout_amd/build.py "
                              f"(hipcc --offload-arch=gfx950); there is no fallback path")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def load_fake():
    """The host core over the recording backend (CPU tests only)."""
    lib = _bind(ctypes.CDLL(FAKE_LIB_PATH))
    lib.afd_fake_log_get.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int]
    lib.afd_fake_set_ends.argtypes = [_P, ctypes.c_int, ctypes.c_uint64]
    lib.afd_fake_tiles.argtypes = [_P, ctypes.c_int]
    lib.afd_fake_set_stall.argtypes = [ctypes.c_int]
    return lib


def check(status, what):
    if status != AFD_OK:
        raise AfdError(status, what)
