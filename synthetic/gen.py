"""Seeded synthetic inputs for the AFD dispatch/combine path.

This module only *draws* inputs: activations, top-k expert ids, routing
weights and FP8 block scales.  It holds none of the exchange's arithmetic
(no counting, no prefix sums, no slot ranks, no reduction), so both the
CPU oracle and the GPU path can consume the same arrays without sharing any
of the computation they are compared on.

Workload shapes follow the afdEP-comm design page ("Result" table: E128,
top-k 8, capacity 2,048, hidden 2,048/4,096, random and skewed routing,
BF16 and FP8 dispatch; E96 for the 1A:3F layout) and the API contract page
("Roles and tensors": ids unique per token in [0, E) or -1, FP32 weights,
float8_e4m3fn activations with FP32 block-128 scales [T, H/128]).

Draw order per instance (fixed, so a seed names one instance):
  * skewed routing only: ``perm = rng.permutation(E)`` first;
  * then for each source s in order: x (standard normal float32 [T, H]),
    the ids, the -1 mask (only when p > 0), the logits (standard normal
    float32 [T, K]).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np

BF16 = "bf16"
FP8 = "fp8"


# --------------------------------------------------------------------------
# Number formats used to *create* inputs (the library itself never converts).
# --------------------------------------------------------------------------

def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even).

    bfloat16 keeps the upper 16 bits of the IEEE binary32 pattern; rounding
    adds 0x7FFF plus the lowest kept bit before truncating.  NaN maps to the
    quiet pattern 0x7FC0 (never produced by normal draws)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """Values of the float8_e4m3fn codes 0x00..0x7E (1 sign, 4 exponent,
    3 mantissa bits, bias 7, no infinities, 0x7F/0xFF are NaN).  Codes
    0x01..0x07 are subnormal with step 2^-9; the largest finite is 448."""
    vals = np.zeros(0x7F, dtype=np.float64)
    for code in range(0x7F):
        e = code >> 3
        m = code & 7
        if e == 0:
            vals[code] = m * 2.0 ** -9
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_table()


def e4m3_bits_to_f32(q: np.ndarray) -> np.ndarray:
    """Decode float8_e4m3fn bytes to float32 (exact; NaN codes give NaN)."""
    q = np.asarray(q, dtype=np.uint8)
    mag = np.full(q.shape, np.nan, dtype=np.float64)
    c = q & 0x7F
    fin = c != 0x7F
    mag[fin] = _E4M3_POS[c[fin]]
    sign = np.where((q & 0x80) != 0, -1.0, 1.0)
    return (sign * mag).astype(np.float32)


def f32_to_e4m3_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 to float8_e4m3fn, nearest with ties to the even code.

    Inputs must satisfy |v| <= 464 (values in (448, 464] round down to 448,
    the largest finite); the block scaling used here keeps |v| <= 448 up to
    one float32 rounding, so no input ever needs saturation or NaN."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    if np.any(~np.isfinite(a)) or np.any(a > 464.0):
        raise ValueError("value outside the e4m3 rounding range")
    tab = _E4M3_POS
    hi = np.searchsorted(tab, a, side="left")          # tab[hi-1] < a <= tab[hi]
    hi = np.minimum(hi, len(tab) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - tab[lo]
    d_hi = tab[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a >= tab[-1], len(tab) - 1, np.where(pick_hi, hi, lo))
    code = code.astype(np.uint8)
    neg = np.signbit(v)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return code


# --------------------------------------------------------------------------
# Instances
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Config:
    name: str
    seed: int
    T: List[int]              # tokens per Attention source
    H: int
    E: int
    F: int
    K: int
    alpha: int
    dtype: str = BF16
    routing: str = "uniform"  # "uniform" | "zipf"
    p_skip: float = 0.0       # probability that a choice is replaced by -1
    bucket: int = 2048
    capacity: int = 2048

    @property
    def N(self) -> int:
        return len(self.T)


@dataclasses.dataclass
class Source:
    x: np.ndarray                 # uint16 [T, H] (bf16 bits) or uint8 [T, H] (e4m3 bits)
    ids: np.ndarray               # int32 [T, K]
    weights: np.ndarray           # float32 [T, K]
    scale: Optional[np.ndarray]   # float32 [T, H/128] (FP8 only)


@dataclasses.dataclass
class Instance:
    cfg: Config
    sources: List[Source]

    def digests(self) -> dict:
        out = {}
        for s, src in enumerate(self.sources):
            for k in ("x", "ids", "weights", "scale"):
                a = getattr(src, k)
                if a is not None:
                    out[f"s{s}.{k}"] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
        return out


def _uniform_ids(rng, T, E, K):
    """K distinct experts per token, uniform without replacement: the first
    K columns of a random permutation per row."""
    if T == 0:
        return np.zeros((0, K), dtype=np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


def _zipf_ids(rng, T, E, K, perm):
    """K distinct experts per token drawn without replacement from a
    Zipf(s=1) popularity over the permuted expert order (expert perm[r] has
    weight 1/(r+1)).  Gumbel-top-k: the K largest of log p + Gumbel noise,
    in descending key order, equals successive sampling without
    replacement."""
    p = np.empty(E, dtype=np.float64)
    p[perm] = 1.0 / np.arange(1, E + 1, dtype=np.float64)
    p /= p.sum()
    if T == 0:
        return np.zeros((0, K), dtype=np.int32)
    keys = np.log(p)[None, :] + rng.gumbel(size=(T, E))
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def _softmax_f32(logits):
    """Per-token softmax over all K logits, in float64, cast to float32.
    Masked (-1) choices keep their weight; nothing is renormalised."""
    z = logits.astype(np.float64)
    if z.shape[0] == 0:
        return z.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def quantize_fp8_blocks(x: np.ndarray):
    """Per 128-column block: scale = float32(amax) / 448, q = e4m3(x / scale)
    computed in float32.  A block of zeros gets scale 1 and codes 0."""
    T, H = x.shape
    xb = x.reshape(T, H // 128, 128)
    amax = np.abs(xb).max(axis=2).astype(np.float32) if T else np.zeros((0, H // 128), np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = f32_to_e4m3_bits((xb / scale[:, :, None]).astype(np.float32)).reshape(T, H)
    return q, scale


def generate(cfg: Config, rng: Optional[np.random.Generator] = None) -> Instance:
    if rng is None:
        rng = np.random.default_rng(cfg.seed)
    perm = rng.permutation(cfg.E) if cfg.routing == "zipf" else None
    sources = []
    for T in cfg.T:
        x = rng.standard_normal((T, cfg.H), dtype=np.float32)
        if cfg.routing == "zipf":
            ids = _zipf_ids(rng, T, cfg.E, cfg.K, perm)
        else:
            ids = _uniform_ids(rng, T, cfg.E, cfg.K)
        if cfg.p_skip > 0:
            mask = rng.random((T, cfg.K)) < cfg.p_skip
            ids = np.where(mask, -1, ids).astype(np.int32)
        logits = rng.standard_normal((T, cfg.K), dtype=np.float32)
        w = _softmax_f32(logits)
        if cfg.dtype == FP8:
            q, scale = quantize_fp8_blocks(x)
            sources.append(Source(q, np.ascontiguousarray(ids), w, scale))
        else:
            sources.append(Source(f32_to_bf16_bits(x), np.ascontiguousarray(ids), w, None))
    return Instance(cfg, sources)


# The five seeded workloads (shapes of the afdEP-comm result table).
def cfg_tiny():
    return Config("tiny", 0, [8], 256, 8, 2, 2, 1, BF16, "uniform", 0.1, 8, 8)


def cfg_decode():
    return Config("2a2f_decode", 1, [128, 128], 2048, 128, 2, 8, 64, BF16, "uniform", 0.0)


def cfg_skew():
    return Config("2a2f_skew_h4096", 2, [512, 512], 4096, 128, 2, 8, 128, BF16, "zipf", 0.0)


def cfg_fp8():
    return Config("2a2f_fp8_prefill", 3, [2048, 2048], 2048, 128, 2, 8, 128, FP8, "uniform", 0.0)


def cfg_ratio_pair():
    """1A:3F then 3A:1F at E96, both drawn from one seed-4 stream."""
    a = Config("1a3f_e96", 4, [2048], 2048, 96, 3, 8, 128, BF16, "uniform", 0.05)
    b = Config("3a1f_e96_view", 4, [2048, 2048, 2048], 2048, 96, 1, 8, 128, BF16, "uniform", 0.05)
    return a, b


def all_instances():
    """Every seeded workload, in order: tiny, decode, skew, fp8, 1A:3F, 3A:1F."""
    out = [generate(cfg_tiny()), generate(cfg_decode()), generate(cfg_skew()), generate(cfg_fp8())]
    a, b = cfg_ratio_pair()
    rng = np.random.default_rng(4)
    out.append(generate(a, rng))
    out.append(generate(b, rng))
    return out


def instance_by_name(name: str) -> Instance:
    if name == "tiny":
        return generate(cfg_tiny())
    if name == "2a2f_decode":
        return generate(cfg_decode())
    if name == "2a2f_skew_h4096":
        return generate(cfg_skew())
    if name == "2a2f_fp8_prefill":
        return generate(cfg_fp8())
    if name in ("1a3f_e96", "3a1f_e96_view"):
        a, b = cfg_ratio_pair()
        rng = np.random.default_rng(4)
        ia = generate(a, rng)
        if name == "1a3f_e96":
            return ia
        return generate(b, rng)
    raise KeyError(name)


WORKLOADS = ["tiny", "2a2f_decode", "2a2f_skew_h4096", "2a2f_fp8_prefill", "1a3f_e96", "3a1f_e96_view"]


def random_small(seed: int, *, N=None, F=None, E=None, K=None, alpha=None, H=256,
                 T=None, p_skip=None, dtype=BF16, bucket=None) -> Instance:
    """A tiny random instance for sweeps (all shape parameters drawn from the
    seed unless given)."""
    rng = np.random.default_rng(1000 + seed)
    F = F if F is not None else int(rng.integers(1, 4))
    E = E if E is not None else F * int(rng.integers(1, 5))
    K = K if K is not None else int(rng.integers(1, min(4, E) + 1))
    N = N if N is not None else int(rng.integers(1, 4))
    alpha = alpha if alpha is not None else int(rng.choice([1, 2, 3, 8]))
    if T is None:
        T = [int(rng.choice([0, 1, 5, 64, 65])) for _ in range(N)]
    p_skip = p_skip if p_skip is not None else float(rng.choice([0.0, 0.2]))
    bucket = bucket if bucket is not None else max(max(T), 1)
    cfg = Config(f"rand{seed}", seed, list(T), H, E, F, K, alpha, dtype, "uniform", p_skip, bucket, bucket)
    return generate(cfg, rng)
