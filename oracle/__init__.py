"""CPU oracle for the AFD dispatch/combine path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library never does, and shares no code with it.

The arithmetic lives in ``afd_oracle.c`` (plain single-threaded C, built with
``-ffp-contract=off``); this module only builds it and marshals numpy arrays.
Each C function names the passage of the afdEP-comm pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "afd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
# the same source built with -fopenmp: the row copy and the combine on
# several threads, for the benchmark's all-cores CPU baseline only
_OMP_LIB_PATH = os.path.join(_HERE, "_build", "liboracle_omp.so")
_lib = None
_serial_lib = None

ROUTE_RANGE, ROUTE_NEG, ROUTE_DUP = 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, no contraction of a*b+c), and
    its OpenMP timing build."""
    if not force and os.path.exists(_LIB_PATH) and os.path.exists(_OMP_LIB_PATH):
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    for path, extra in ((_LIB_PATH, ["-Wno-unknown-pragmas"]), (_OMP_LIB_PATH, ["-fopenmp"])):
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-Werror", *extra, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, path)
    return _LIB_PATH


def lib():
    global _lib, _serial_lib
    if _lib is None:
        # AFD_ORACLE_LIB loads another build of the same source instead (the
        # sanitizer test's AddressSanitizer/UBSan build); build() never
        # writes it
        path = os.environ.get("AFD_ORACLE_LIB")
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path):
                build()
        _serial_lib = _lib = ctypes.CDLL(path)
    return _lib


def set_parallel(on: bool) -> int:
    """Run the following calls on the OpenMP timing build (on=True) or the
    plain single-threaded build; returns the threads the row copy and the
    combine use.  Benchmark only: the tests use the plain build."""
    global _lib
    lib()
    if on:
        if not os.path.exists(_OMP_LIB_PATH):
            build()
        _lib = ctypes.CDLL(_OMP_LIB_PATH)
    else:
        _lib = _serial_lib
    return int(_lib.orc_threads())


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ptr_array(arrs: Sequence[np.ndarray]):
    t = ctypes.c_void_p * max(len(arrs), 1)
    return t(*[a.ctypes.data for a in arrs])


class Layout:
    """Result of :func:`layout` (all numpy)."""

    def __init__(self, ends, host_counts, rows_exact, slot_part, slot_row, err):
        self.ends = ends                # int32 [E]
        self.host_counts = host_counts  # int32 [E]
        self.rows_exact = rows_exact    # int64 [F]
        self.slot_part = slot_part      # int32 [ntok, K]
        self.slot_row = slot_row        # int32 [ntok, K]
        self.err = err                  # (code, s, t, k)


def check_config(T: Sequence[int], bucket: int, capacity: int, E: int, F: int, K: int, H: int, alpha: int) -> bool:
    """Step one of a round (API contract page, "Roles and tensors"): is the
    configuration with per-source token counts T valid?"""
    T_arr = np.ascontiguousarray(T, dtype=np.int32)
    return lib().orc_check_config(len(T_arr), _p(T_arr), bucket, capacity, E, F, K, H, alpha) == 0


def layout(T: Sequence[int], ids: np.ndarray, E: int, F: int, K: int, alpha: int) -> Layout:
    """ids: int32 [sum(T), K] (sources concatenated in order)."""
    T_arr = np.ascontiguousarray(T, dtype=np.int32)
    ntok = int(T_arr.sum())
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(ntok, K)
    ends = np.zeros(E, np.int32)
    hc = np.zeros(E, np.int32)
    rows = np.zeros(F, np.int64)
    sp = np.zeros((max(ntok, 1), K), np.int32)
    sr = np.zeros((max(ntok, 1), K), np.int32)
    err = np.zeros(4, np.int32)
    rc = lib().orc_layout(len(T_arr), _p(T_arr), _p(ids), E, F, K, alpha, _p(ends), _p(hc),
                          _p(rows), _p(sp), _p(sr), _p(err))
    if rc != 0:
        raise ValueError("invalid configuration")
    return Layout(ends, hc, rows, sp[:ntok], sr[:ntok], tuple(int(v) for v in err))


def dispatch(x_all: np.ndarray, w_all: np.ndarray, lay: Layout, F: int, rows_cap: Sequence[int],
             fill_rows: Optional[int] = None, out=None):
    """Expert-major rows and per-row weights for every partition.

    x_all: [ntok, H] uint16 (bf16 bits) or uint8 (e4m3 bits).  Rows that are
    not targets keep ``fill_rows`` bytes (0 if None) and weight NaN.  With
    ``out`` = (rows, roww) from an earlier call, those arrays are written
    again in place (rows that are not targets keep what they held)."""
    ntok, K = lay.slot_part.shape
    x_all = np.ascontiguousarray(x_all)
    row_bytes = x_all.shape[1] * x_all.itemsize if ntok else 0
    if out is not None:
        rows, roww = out
    else:
        rows = [np.full((rows_cap[f], x_all.shape[1]), fill_rows or 0, dtype=x_all.dtype) for f in range(F)]
        roww = [np.full(rows_cap[f], np.nan, np.float32) for f in range(F)]
    if ntok:
        lib().orc_dispatch(ctypes.c_int64(ntok), K, _p(x_all), ctypes.c_int64(row_bytes),
                           _p(np.ascontiguousarray(w_all, np.float32)), _p(lay.slot_part),
                           _p(lay.slot_row), _ptr_array(rows), _ptr_array(roww))
    return rows, roww


def dispatch_scales(T: Sequence[int], scale_src: List[np.ndarray], strides: List[tuple], G: int,
                    lay: Layout, F: int, rows_cap: Sequence[int], out=None):
    """scale_src[s]: float32 buffer of source s; strides[s] = (stride_t, stride_g) in elements.
    ``out``: scale arrays of an earlier call, written again in place."""
    T_arr = np.ascontiguousarray(T, dtype=np.int32)
    ntok, K = lay.slot_part.shape
    scales = out if out is not None else [np.full((rows_cap[f], G), np.nan, np.float32) for f in range(F)]
    st = np.ascontiguousarray([s[0] for s in strides], np.int64)
    sg = np.ascontiguousarray([s[1] for s in strides], np.int64)
    srcs = [np.ascontiguousarray(a, np.float32) if a is not None else np.zeros(1, np.float32) for a in scale_src]
    if ntok:
        lib().orc_dispatch_scales(len(T_arr), _p(T_arr), K, G, _ptr_array(srcs), _p(st), _p(sg),
                                  _p(lay.slot_part), _p(lay.slot_row), _ptr_array(scales))
    return scales


def identity_experts(fp8: bool, E: int, F: int, f: int, alpha: int, H: int, ends: np.ndarray,
                     rows: np.ndarray, scales: Optional[np.ndarray], y: np.ndarray) -> np.ndarray:
    """Fill y (uint16 [rows, H]) in place for partition f's live rows."""
    ends = np.ascontiguousarray(ends, np.int32)
    sc = np.ascontiguousarray(scales, np.float32) if scales is not None else np.zeros(1, np.float32)
    lib().orc_identity_experts(1 if fp8 else 0, E, F, f, alpha, H, _p(ends),
                               _p(np.ascontiguousarray(rows)), _p(sc), _p(y))
    return y


def combine(w_all: np.ndarray, lay: Layout, H: int, ys: List[np.ndarray], out=None) -> np.ndarray:
    """``out``: a uint16 [ntok, H] array of an earlier call, overwritten."""
    ntok, K = lay.slot_part.shape
    if out is None:
        out = np.zeros((ntok, H), np.uint16)
    if ntok:
        ys = [np.ascontiguousarray(y, np.uint16) for y in ys]
        lib().orc_combine(ctypes.c_int64(ntok), K, H, _p(np.ascontiguousarray(w_all, np.float32)),
                          _p(lay.slot_part), _p(lay.slot_row), _ptr_array(ys), _p(out))
    return out


# ---- per-stage combine (design page, sections 6 and 19) ----

COMBINE_ONCE, COMBINE_PER_STAGE, COMBINE_PER_STAGE_FP8 = "once", "per_stage", "per_stage_fp8"


def fp8_row_bytes(H: int) -> int:
    """Bytes of one FP8 partial row: H codes, H/128 scale bytes, padding to 32."""
    lib().orc_fp8_row_bytes.restype = ctypes.c_int64
    return int(lib().orc_fp8_row_bytes(H))


def combine_partials(w_all: np.ndarray, lay: Layout, H: int, F: int, ys: List[np.ndarray]):
    """Stage one: BF16 partial [F, ntok, H] of every partition and token, and
    has [F, ntok] (1 where the token has a live choice in that partition;
    other rows stay 0)."""
    ntok, K = lay.slot_part.shape
    partial = np.zeros((F, ntok, H), np.uint16)
    has = np.zeros((F, ntok), np.uint8)
    if ntok:
        ys = [np.ascontiguousarray(y, np.uint16) for y in ys]
        lib().orc_combine_partials(ctypes.c_int64(ntok), K, H, F, _p(np.ascontiguousarray(w_all, np.float32)),
                                   _p(lay.slot_part), _p(lay.slot_row), _ptr_array(ys), _p(partial), _p(has))
    return partial, has


def quantize_fp8_rows(partial_rows: np.ndarray) -> np.ndarray:
    """FP8 form (codes, scale bytes, zero padding) of BF16 rows [n, H]."""
    partial_rows = np.ascontiguousarray(partial_rows, np.uint16)
    n, H = partial_rows.shape
    out = np.zeros((n, fp8_row_bytes(H)), np.uint8)
    for i in range(n):
        lib().orc_quantize_fp8_row(H, _p(partial_rows[i]), _p(out[i]))
    return out


def quantize_partials(partial: np.ndarray, has: np.ndarray) -> np.ndarray:
    """FP8 rows [F, ntok, row bytes] of the partials that exist (others 0)."""
    F, ntok, H = partial.shape
    q = np.zeros((F, ntok, fp8_row_bytes(H)), np.uint8)
    for f in range(F):
        idx = np.nonzero(has[f])[0]
        if len(idx):
            q[f, idx] = quantize_fp8_rows(partial[f, idx])
    return q


def combine_stages(lay: Layout, H: int, partial: Optional[np.ndarray], qrows: Optional[np.ndarray]) -> np.ndarray:
    """Stage two: the BF16 result [ntok, H] from the BF16 partials
    (qrows None) or from their FP8 rows."""
    ntok, K = lay.slot_part.shape
    out = np.zeros((ntok, H), np.uint16)
    if ntok:
        fp8 = qrows is not None
        pa = np.ascontiguousarray(partial if partial is not None else np.zeros(1), np.uint16)
        qa = np.ascontiguousarray(qrows if fp8 else np.zeros(1), np.uint8)
        lib().orc_combine_stages(ctypes.c_int64(ntok), K, H, 1 if fp8 else 0, _p(lay.slot_part), _p(pa), _p(qa),
                                 _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib().orc_e4m3_encode(_p(v), _p(out), ctypes.c_int64(v.size))
    return out


def bf16_round(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.zeros(v.shape, np.uint16)
    lib().orc_bf16_round(_p(v), _p(out), ctypes.c_int64(v.size))
    return out


def e4m3_decode(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    out = np.zeros(q.shape, np.float32)
    lib().orc_e4m3_decode(_p(q), _p(out), ctypes.c_int64(q.size))
    return out


class RoundResult:
    def __init__(self, lay, rows, roww, scales, ys, out, rows_cap, partial=None, has=None, qrows=None):
        self.layout = lay
        self.rows = rows
        self.row_weights = roww
        self.scales = scales
        self.replies = ys
        self.out = out          # uint16 [ntok, H]
        self.rows_cap = rows_cap
        self.partial = partial  # per-stage combine: uint16 [F, ntok, H]
        self.has = has          # uint8 [F, ntok]
        self.qrows = qrows      # FP8 partial rows: uint8 [F, ntok, row bytes]


def run_round(inst, rows_cap: Optional[Sequence[int]] = None, combine_mode: str = COMBINE_ONCE) -> RoundResult:
    """The whole round for a generated instance (synthetic.gen.Instance):
    layout -> dispatch (+scales) -> identity experts -> combine, the combine
    rounding once (COMBINE_ONCE) or once per stage with BF16 or FP8
    partials."""
    cfg = inst.cfg
    fp8 = cfg.dtype == "fp8"
    T = [len(s.ids) for s in inst.sources]
    K, H, E, F = cfg.K, cfg.H, cfg.E, cfg.F
    if not check_config(T, cfg.bucket, cfg.capacity, E, F, K, H, cfg.alpha):
        raise ValueError("invalid configuration or shapes")
    ids = np.concatenate([s.ids for s in inst.sources]) if sum(T) else np.zeros((0, K), np.int32)
    w = np.concatenate([s.weights for s in inst.sources]) if sum(T) else np.zeros((0, K), np.float32)
    dt = np.uint8 if fp8 else np.uint16
    x = np.concatenate([s.x for s in inst.sources]) if sum(T) else np.zeros((0, H), dt)
    lay = layout(T, ids, E, F, K, cfg.alpha)
    if rows_cap is None:
        rows_cap = [int(max(lay.rows_exact[f], 1)) for f in range(F)]
    rows, roww = dispatch(x, w, lay, F, rows_cap)
    scales = None
    if fp8:
        scales = dispatch_scales(T, [s.scale for s in inst.sources], [(H // 128, 1)] * len(T), H // 128,
                                 lay, F, rows_cap)
    ys = []
    for f in range(F):
        y = np.zeros((rows_cap[f], H), np.uint16)
        identity_experts(fp8, E, F, f, cfg.alpha, H, lay.ends, rows[f], scales[f] if fp8 else None, y)
        ys.append(y)
    if combine_mode == COMBINE_ONCE:
        return RoundResult(lay, rows, roww, scales, ys, combine(w, lay, H, ys), rows_cap)
    partial, has = combine_partials(w, lay, H, F, ys)
    qrows = quantize_partials(partial, has) if combine_mode == COMBINE_PER_STAGE_FP8 else None
    out = combine_stages(lay, H, None if qrows is not None else partial, qrows)
    return RoundResult(lay, rows, roww, scales, ys, out, rows_cap, partial, has, qrows)
