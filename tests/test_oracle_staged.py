"""Pins for the oracle's per-stage combine (CPU).

The per-stage combine follows the afdEP-comm design page: with more than
one FFN domain each FFN's partial is rounded to BF16 before the sum over
domains (section 6), and the opt-in FP8 replies carry each partial as
E4M3 codes with one power-of-two scale per 128 elements (section 19):
e is the smallest integer with amax <= 448 * 2^e, at least -117; the
source dequantises, sums in float32 in slot order (ascending last top-k
lane per domain) and rounds once.

What pins it, independently of the oracle's own mechanism:
  * the E4M3 encoder against torch's float8_e4m3fn cast (every tie between
    adjacent codes, every code, random values in every binade);
  * scale exponents against the closed form ceil(log2(amax / 448)) from
    frexp, and the page's special values (clamp at -117, 2^120 for an
    infinite amax);
  * quantised rows against torch's cast of the exactly scaled values, and
    the section 19 error bound (|decoded - v| <= amax_group / 16);
  * stage one against the pinned single-rounding combine run on the layout
    with other partitions' choices skipped;
  * stage two against the pinned single-rounding combine of the partials
    (weight 1, one row per partition, in last-lane order);
  * the summation order against hand-derived values where every other
    plausible order gives a different result;
  * closed forms with identity experts within the bound of three BF16
    roundings (plus the FP8 bound), exact results when every partial is a
    short integer, and F = 1 reducing to the single-rounding combine."""
import math

import numpy as np
import pytest

import oracle
from synthetic import gen

ATOL, RTOL = 1e-3, 1e-2
WORKLOADS = ["tiny", "2a2f_decode", "1a3f_e96"]


def _concat(inst, attr):
    arrs = [getattr(s, attr) for s in inst.sources]
    return np.concatenate(arrs) if sum(a.shape[0] for a in arrs) else arrs[0]


def _torch_e4m3(v32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_value(q: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _exponent_ref(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (closed form), at least -117;
    the page's top scale 2^120 for an infinite amax."""
    if math.isinf(amax):
        return 120
    if amax == 0.0:
        return -117
    m, x = math.frexp(amax / 448.0)          # amax / 448 = m * 2^x, m in [0.5, 1)
    e = x - 1 if m == 0.5 else x
    return max(e, -117)


# ---------------------------------------------------------------- formats ----

def test_e4m3_encoder_matches_torch():
    pos = _torch_e4m3_value(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)   # codes 0..126
    mids = (pos[:-1] + pos[1:]) / 2.0                                                # every tie
    rng = np.random.default_rng(21)
    rand = np.concatenate([rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-12, 9, 20000),
                           rng.uniform(-448, 448, 5000)])
    near = np.concatenate([pos * (1 + 2.0 ** -20), pos * (1 - 2.0 ** -20), mids * (1 + 2.0 ** -22),
                           mids * (1 - 2.0 ** -22)])
    v = np.concatenate([pos, -pos, mids, -mids, rand, near, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))
    # the page's readings at the edges: NaN keeps its element, infinity saturates
    # to 448 (so that 448 * 2^120 decodes to infinity)
    sp = oracle.e4m3_encode(np.array([np.nan, np.inf, -np.inf], np.float32))
    assert sp[0] & 0x7F == 0x7F and sp[1] == 0x7E and sp[2] == 0xFE


def _rows_with_groups(rng, n, H):
    """BF16 rows whose 128-element groups span the exponent range, plus the
    page's special groups."""
    G = H // 128
    v = rng.standard_normal((n, G, 128)) * 2.0 ** rng.integers(-135, 118, (n, G, 1))
    v = v.reshape(n, H).astype(np.float32)
    rows = gen.f32_to_bf16_bits(v)
    specials = []
    bf = lambda a: gen.f32_to_bf16_bits(np.asarray(a, np.float32))
    z = np.zeros(128, np.float32)
    specials.append(bf(z))                                           # amax 0 -> clamp
    specials.append(np.full(128, 0x0001, np.uint16))                 # smallest subnormal
    for k in (-117, -116, -20, 0, 3, 119):
        g = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** (k + 5))
        g[7] = np.float32(448.0 * 2.0 ** k)                          # amax exactly 448 * 2^k
        g = np.clip(g, -448.0 * 2.0 ** k, 448.0 * 2.0 ** k)
        specials.append(bf(g))
        g2 = g.copy()
        g2[7] = np.float32(448.0 * 2.0 ** k * (1 + 2.0 ** -7))       # just above: one more
        specials.append(bf(g2))
    top = rng.standard_normal(128).astype(np.float32)
    top[3] = 3.3895314e38                                            # largest finite BF16
    specials.append(bf(top))
    nan = rng.standard_normal(128).astype(np.float32)
    nan[5] = np.nan
    specials.append(bf(nan))
    inf = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** 112)
    inf[9] = np.inf
    inf[10] = np.float32(2.0 ** 111)
    specials.append(bf(inf))
    sp = np.concatenate(specials)
    sp = np.concatenate([sp, np.zeros((-len(sp)) % H, np.uint16)]).reshape(-1, H)
    return np.concatenate([rows, sp])


@pytest.mark.parametrize("H", [256, 2048])
def test_quantized_rows_match_torch_and_closed_form(H):
    rng = np.random.default_rng(22 + H)
    rows = _rows_with_groups(rng, 24, H)
    q = oracle.quantize_fp8_rows(rows)
    G = H // 128
    rb = oracle.fp8_row_bytes(H)
    assert q.shape == (rows.shape[0], rb) and rb == H + (G + 31) // 32 * 32 and rb % 16 == 0
    assert np.all(q[:, H + G:] == 0)
    vals = gen.bf16_bits_to_f32(rows).reshape(-1, G, 128)
    for i in range(rows.shape[0]):
        for b in range(G):
            grp = vals[i, b]
            fin = grp[~np.isnan(grp)]
            amax = float(np.abs(fin).max()) if fin.size else 0.0
            e = _exponent_ref(amax)
            assert q[i, H + b] == 127 + e, (i, b, amax)
            codes = q[i, b * 128:(b + 1) * 128]
            scaled = np.ldexp(grp.astype(np.float32), -e).astype(np.float32)
            ok = np.isfinite(scaled)
            assert np.array_equal(codes[ok], _torch_e4m3(scaled[ok])), (i, b)
            assert np.all(codes[np.isnan(grp)] & 0x7F == 0x7F)
            infs = np.isinf(grp)
            if infs.any():
                assert e == 120
                dec = _torch_e4m3_value(codes[infs]).astype(np.float64) * 2.0 ** e
                assert np.all(dec > np.finfo(np.float32).max)        # overflows float32: infinity


def test_quantization_error_bound():
    """Design page, section 19 error bound: |decoded - v| <= amax_group / 16
    for every element; a value that is already representable round-trips."""
    rng = np.random.default_rng(23)
    H = 1024
    v = (rng.standard_normal((64, H)) * 2.0 ** rng.integers(-40, 40, (64, 1))).astype(np.float32)
    rows = gen.f32_to_bf16_bits(v)
    q = oracle.quantize_fp8_rows(rows)
    x = gen.bf16_bits_to_f32(rows).astype(np.float64).reshape(64, H // 128, 128)
    sf = q[:, H:H + H // 128].astype(np.int64) - 127
    dq = _torch_e4m3_value(q[:, :H]).astype(np.float64).reshape(64, H // 128, 128) * 2.0 ** sf[:, :, None]
    amax = np.abs(x).max(axis=2, keepdims=True)
    assert np.all(np.abs(dq - x) <= 2.0 ** -4 * amax)
    # the dequantised values are representable: quantising them again keeps
    # every value (the scale may drop by one when the amax rounded down)
    rt = oracle.quantize_fp8_rows(gen.f32_to_bf16_bits(dq.reshape(64, H).astype(np.float32)))
    sf2 = rt[:, H:H + H // 128].astype(np.int64) - 127
    dq2 = _torch_e4m3_value(rt[:, :H]).astype(np.float64).reshape(64, H // 128, 128) * 2.0 ** sf2[:, :, None]
    assert np.array_equal(dq2, dq)


# ------------------------------------------------------------ stage one ----

def _masked(lay, f):
    sp = np.where(lay.slot_part == f, lay.slot_part, -1).astype(np.int32)
    sr = np.where(lay.slot_part == f, lay.slot_row, -1).astype(np.int32)
    return oracle.Layout(lay.ends, lay.host_counts, lay.rows_exact, sp, sr, lay.err)


def _cases():
    out = [gen.instance_by_name(n) for n in WORKLOADS]
    out.append(gen.random_small(31, N=3, F=3, E=9, K=3, alpha=2, T=[17, 0, 30], H=256, p_skip=0.2))
    out.append(gen.random_small(32, N=2, F=4, E=8, K=4, alpha=3, T=[65, 5], H=512, p_skip=0.2, dtype="fp8"))
    return out


@pytest.mark.parametrize("i", range(5))
def test_partials_equal_masked_single_rounding_combine(i):
    inst = _cases()[i]
    cfg = inst.cfg
    r = oracle.run_round(inst, combine_mode=oracle.COMBINE_PER_STAGE)
    w = _concat(inst, "weights")
    for f in range(cfg.F):
        m = _masked(r.layout, f)
        ref = oracle.combine(w, m, cfg.H, r.replies)
        has = (r.layout.slot_part == f).any(axis=1)
        assert np.array_equal(r.has[f].astype(bool), has)
        assert np.array_equal(r.partial[f][has], ref[has])
        assert np.all(r.partial[f][~has] == 0)


# ------------------------------------------------------------ stage two ----

def _last_lane_layout(lay, F):
    """One 'choice' per partition holding a partial, ordered by the last live
    top-k lane mapping to it; its row is the token itself."""
    ntok, K = lay.slot_part.shape
    sp = -np.ones((ntok, F), np.int32)
    sr = -np.ones((ntok, F), np.int32)
    for g in range(ntok):
        last = {}
        for k in range(K):
            f = int(lay.slot_part[g, k])
            if f >= 0:
                last[f] = k
        for j, f in enumerate(sorted(last, key=lambda q: last[q])):
            sp[g, j] = f
            sr[g, j] = g
    return oracle.Layout(lay.ends, lay.host_counts, lay.rows_exact, sp, sr, lay.err)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("i", range(5))
def test_stage_two_equals_single_rounding_combine_of_partials(i, fp8):
    inst = _cases()[i]
    cfg = inst.cfg
    mode = oracle.COMBINE_PER_STAGE_FP8 if fp8 else oracle.COMBINE_PER_STAGE
    r = oracle.run_round(inst, combine_mode=mode)
    lay2 = _last_lane_layout(r.layout, cfg.F)
    if fp8:
        H = cfg.H
        vals = []
        for f in range(cfg.F):
            q = r.qrows[f]
            sf = q[:, H:H + H // 128].astype(np.int64) - 127
            v = _torch_e4m3_value(q[:, :H]).astype(np.float64) * 2.0 ** np.repeat(sf, 128, axis=1)
            b = gen.f32_to_bf16_bits(v.astype(np.float32))
            assert np.array_equal(gen.bf16_bits_to_f32(b).astype(np.float64)[r.has[f] == 1], v[r.has[f] == 1])
            vals.append(b)
        rows = vals
    else:
        rows = [r.partial[f] for f in range(cfg.F)]
    ones = np.ones(lay2.slot_part.shape, np.float32)
    ref = oracle.combine(ones, lay2, cfg.H, rows)
    assert np.array_equal(r.out, ref)


def test_stage_two_order_is_last_lane():
    """Partials 1, -1 and 2^-30: the sum is 2^-30 only when the tiny partial
    comes after both others, else +0.  Token A's partitions by lane are
    [1, 0, 2, 1] (last lanes: 0 -> 1, 2 -> 2, 1 -> 3: the tiny partition 2 is in
    the middle, so +0), while ascending partitions or first lanes would add it
    last.  Token B's are [2, 0, 1, 2] (last lanes: 0, 1, then 2: 2^-30), while
    first lanes would add it first."""
    H, E, F, K = 256, 6, 3, 4
    ids = np.array([[2, 0, 4, 3], [4, 0, 2, 5]], np.int32)
    lay = oracle.layout([2], ids, E, F, K, 1)
    w = np.ones((2, K), np.float32)
    val = {0: 1.0, 1: -1.0, 2: 2.0 ** -30}
    caps = [int(max(v, 1)) for v in lay.rows_exact]
    ys = [np.zeros((c, H), np.uint16) for c in caps]
    for g in range(2):
        for k in range(K):
            f, row = int(lay.slot_part[g, k]), int(lay.slot_row[g, k])
            n = int((lay.slot_part[g] == f).sum())           # choices of g in f share its value
            ys[f][row] = gen.f32_to_bf16_bits(np.full(H, val[f] / n, np.float32))
    for mode in (oracle.COMBINE_PER_STAGE, oracle.COMBINE_PER_STAGE_FP8):
        partial, has = oracle.combine_partials(w, lay, H, F, ys)
        assert np.array_equal(gen.bf16_bits_to_f32(partial[:, :, 0]), [[1.0, 1.0], [-1.0, -1.0], [2.0 ** -30] * 2])
        q = oracle.quantize_partials(partial, has) if mode == oracle.COMBINE_PER_STAGE_FP8 else None
        out = oracle.combine_stages(lay, H, None if q is not None else partial, q)
        assert np.all(out[0] == 0x0000)
        assert np.all(gen.bf16_bits_to_f32(out[1]) == np.float32(2.0 ** -30))


# ---------------------------------------------------------- closed forms ----

def _xhat(inst):
    x = _concat(inst, "x")
    if inst.cfg.dtype == "fp8":
        sc = _concat(inst, "scale")
        return gen.e4m3_bits_to_f32(x).astype(np.float64) * np.repeat(sc.astype(np.float64), 128, axis=1)
    return gen.bf16_bits_to_f32(x).astype(np.float64)


@pytest.mark.parametrize("name", WORKLOADS)
@pytest.mark.parametrize("fp8", [False, True])
def test_staged_closed_form(name, fp8):
    """Identity experts: out[t] = sum_k w_k s_{e_k} x[t], within three BF16
    roundings of same-sign terms, plus 2^-4 of each partial's group amax for
    FP8 partials (design page, section 19)."""
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    r = oracle.run_round(inst, combine_mode=oracle.COMBINE_PER_STAGE_FP8 if fp8 else oracle.COMBINE_PER_STAGE)
    ids = _concat(inst, "ids")
    w = _concat(inst, "weights").astype(np.float64)
    live = r.layout.slot_part >= 0
    coef = np.where(live, w * (1.0 + ids.astype(np.float64) / cfg.E), 0.0).sum(axis=1)
    ref = coef[:, None] * _xhat(inst)
    got = gen.bf16_bits_to_f32(r.out).astype(np.float64)
    bound = 3.03 * 2.0 ** -8 * np.abs(ref)
    if fp8:
        ntok = ref.shape[0]
        for f in range(cfg.F):
            p = np.abs(gen.bf16_bits_to_f32(r.partial[f]).astype(np.float64)).reshape(ntok, -1, 128)
            bound = bound + np.repeat(p.max(axis=2), 128, axis=1) * 2.0 ** -4 * (1 + 2.0 ** -7)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref)) or fp8


def test_fp8_partials_exact_for_short_integers():
    """Every partial a small integer (at most 4 significant bits): FP8 partials
    are exact, and both per-stage results equal the exact integer sum."""
    rng = np.random.default_rng(24)
    H, E, F, K, T = 256, 12, 3, 3, 40
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    lay = oracle.layout([T], ids, E, F, K, 2)
    w = np.ones((T, K), np.float32)
    caps = [int(max(v, 1)) for v in lay.rows_exact]
    ints = [rng.integers(-3, 4, (c, H)) for c in caps]
    ys = [gen.f32_to_bf16_bits(a.astype(np.float32)) for a in ints]
    exact = np.zeros((T, H), np.int64)
    for g in range(T):
        for k in range(K):
            exact[g] += ints[lay.slot_part[g, k]][lay.slot_row[g, k]]
    partial, has = oracle.combine_partials(w, lay, H, F, ys)
    q = oracle.quantize_partials(partial, has)
    o_bf = oracle.combine_stages(lay, H, partial, None)
    o_f8 = oracle.combine_stages(lay, H, None, q)
    want = gen.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.array_equal(o_bf, want) and np.array_equal(o_f8, want)


def test_single_partition_reduces_to_single_rounding():
    for seed in range(4):
        inst = gen.random_small(40 + seed, F=1, H=256)
        a = oracle.run_round(inst)
        b = oracle.run_round(inst, combine_mode=oracle.COMBINE_PER_STAGE)
        assert np.array_equal(a.out, b.out)
