"""Pins for the oracle's dispatch rows, identity experts and combine (CPU).

  * rows/scales/weights: copy semantics checked by numpy fancy indexing;
  * identity experts: float32 numpy products rounded by the generator's own
    bf16 rounding (itself pinned to torch);
  * combine: the float64 closed form out[t] = sum_k w_k * s_{e_k} * x[t]
    with identity experts; a scipy.sparse routing-matrix product for
    arbitrary replies; exact special cases (K = 1 and w = 1, one live
    choice, all skipped, doubling); padding rows never read.
The tolerance is the one stated for the combine: 1e-3 absolute plus 1e-2
relative per element."""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from synthetic import gen

ATOL, RTOL = 1e-3, 1e-2


def _concat(inst, attr):
    arrs = [getattr(s, attr) for s in inst.sources]
    return np.concatenate(arrs) if sum(a.shape[0] for a in arrs) else arrs[0]


def _xhat(inst):
    """float64 value of each token's activation row."""
    x = _concat(inst, "x")
    if inst.cfg.dtype == "fp8":
        sc = _concat(inst, "scale")
        return gen.e4m3_bits_to_f32(x).astype(np.float64) * np.repeat(sc.astype(np.float64), 128, axis=1)
    return gen.bf16_bits_to_f32(x).astype(np.float64)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_rows_scales_weights_are_copies(name):
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    r = oracle.run_round(inst)
    x = _concat(inst, "x")
    w = _concat(inst, "weights")
    g, k = np.nonzero(r.layout.slot_part >= 0)
    f = r.layout.slot_part[g, k]
    row = r.layout.slot_row[g, k]
    for fi in range(cfg.F):
        m = f == fi
        assert np.array_equal(r.rows[fi][row[m]], x[g[m]])
        assert np.array_equal(r.row_weights[fi][row[m]], w[g[m], k[m]])
        if cfg.dtype == "fp8":
            sc = _concat(inst, "scale")
            assert np.array_equal(r.scales[fi][row[m]], sc[g[m]])


def test_strided_scales_equal_dense():
    inst = gen.random_small(3, N=2, F=2, E=8, K=3, alpha=4, T=[7, 5], dtype="fp8", H=512)
    cfg = inst.cfg
    ids = _concat(inst, "ids")
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    caps = [int(max(v, 1)) for v in lay.rows_exact]
    G = cfg.H // 128
    dense = oracle.dispatch_scales(cfg.T, [s.scale for s in inst.sources], [(G, 1)] * 2, G, lay, 2, caps)
    # column-major copies: element (t, b) at b * T + t
    cm = [np.ascontiguousarray(s.scale.T).ravel() for s in inst.sources]
    strided = oracle.dispatch_scales(cfg.T, cm, [(1, T) for T in cfg.T], G, lay, 2, caps)
    for a, b in zip(dense, strided):
        assert np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_identity_experts_bit_exact(name):
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    r = oracle.run_round(inst)
    E_loc = cfg.E // cfg.F
    for f in range(cfg.F):
        prev = 0
        for j in range(E_loc):
            e = f * E_loc + j
            st = (prev + cfg.alpha - 1) // cfg.alpha * cfg.alpha
            en = int(r.layout.ends[e])
            se = np.float32(1.0) + np.float32(e) / np.float32(cfg.E)
            if en > st:
                if cfg.dtype == "fp8":
                    xv = gen.e4m3_bits_to_f32(r.rows[f][st:en]) * np.repeat(r.scales[f][st:en], 128, axis=1)
                else:
                    xv = gen.bf16_bits_to_f32(r.rows[f][st:en])
                expect = gen.f32_to_bf16_bits((xv.astype(np.float32) * se).astype(np.float32))
                assert np.array_equal(r.replies[f][st:en], expect)
            prev = en


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_combine_closed_form(name):
    """With identity experts, out[t] = sum_k w_k * s_{e_k} * x[t]."""
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    r = oracle.run_round(inst)
    ids = _concat(inst, "ids")
    w = _concat(inst, "weights").astype(np.float64)
    live = r.layout.slot_part >= 0
    s_e = 1.0 + ids.astype(np.float64) / cfg.E
    coef = np.where(live, w * s_e, 0.0).sum(axis=1)
    ref = coef[:, None] * _xhat(inst)
    got = gen.bf16_bits_to_f32(r.out).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))
    # tighter, from the arithmetic: two bf16 roundings of same-sign terms
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)


def test_combine_sparse_routing_matrix_any_replies():
    inst = gen.random_small(11, N=3, F=3, E=9, K=3, alpha=2, T=[17, 0, 30], H=256, p_skip=0.2)
    cfg = inst.cfg
    ids = _concat(inst, "ids")
    w = _concat(inst, "weights")
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    rng = np.random.default_rng(12)
    caps = [int(max(v, 1)) for v in lay.rows_exact]
    ys = [gen.f32_to_bf16_bits(rng.standard_normal((c, cfg.H)).astype(np.float32)) for c in caps]
    out = oracle.combine(w, lay, cfg.H, ys)
    off = np.concatenate([[0], np.cumsum(caps)[:-1]])
    g, k = np.nonzero(lay.slot_part >= 0)
    cols = off[lay.slot_part[g, k]] + lay.slot_row[g, k]
    S = sp.csr_matrix((w[g, k].astype(np.float64), (g, cols)), shape=(ids.shape[0], sum(caps)))
    Y = np.concatenate([gen.bf16_bits_to_f32(y).astype(np.float64) for y in ys])
    ref = S @ Y
    got = gen.bf16_bits_to_f32(out).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def test_combine_exact_special_cases():
    rng = np.random.default_rng(13)
    H = 256
    # (i) K = 1, w = 1: the output is the reply row, bit for bit
    ids = rng.integers(0, 4, (20, 1)).astype(np.int32)
    lay = oracle.layout([20], ids, 4, 2, 1, 1)
    caps = [int(max(v, 1)) for v in lay.rows_exact]
    ys = [gen.f32_to_bf16_bits(rng.standard_normal((c, H)).astype(np.float32)) for c in caps]
    out = oracle.combine(np.ones((20, 1), np.float32), lay, H, ys)
    for g in range(20):
        assert np.array_equal(out[g], ys[lay.slot_part[g, 0]][lay.slot_row[g, 0]])
    # (ii) one live choice of weight w: out = bf16(w * y)
    ids2 = np.array([[-1, 2, -1]] * 5, np.int32)
    w2 = rng.random((5, 3)).astype(np.float32)
    lay2 = oracle.layout([5], ids2, 4, 2, 3, 1)
    ys2 = [gen.f32_to_bf16_bits(rng.standard_normal((max(int(v), 1), H)).astype(np.float32)) for v in lay2.rows_exact]
    out2 = oracle.combine(w2, lay2, H, ys2)
    for g in range(5):
        y = gen.bf16_bits_to_f32(ys2[1][lay2.slot_row[g, 1]])
        assert np.array_equal(out2[g], gen.f32_to_bf16_bits((w2[g, 1] * y).astype(np.float32)))
    # (iii) every choice skipped: +0 exactly
    lay3 = oracle.layout([4], -np.ones((4, 2), np.int32), 4, 2, 2, 1)
    out3 = oracle.combine(rng.random((4, 2)).astype(np.float32), lay3, H, [np.zeros((1, H), np.uint16)] * 2)
    assert np.all(out3 == 0)
    # (iv) doubling every reply doubles the output exactly
    ids4 = np.argsort(rng.random((30, 8)), axis=1)[:, :3].astype(np.int32)
    w4 = rng.random((30, 3)).astype(np.float32)
    lay4 = oracle.layout([30], ids4, 8, 2, 3, 2)
    caps4 = [int(max(v, 1)) for v in lay4.rows_exact]
    ys4 = [gen.f32_to_bf16_bits(rng.standard_normal((c, H)).astype(np.float32)) for c in caps4]
    ys4x2 = [gen.f32_to_bf16_bits(gen.bf16_bits_to_f32(y) * np.float32(2)) for y in ys4]
    o1 = gen.bf16_bits_to_f32(oracle.combine(w4, lay4, H, ys4))
    o2 = gen.bf16_bits_to_f32(oracle.combine(w4, lay4, H, ys4x2))
    assert np.array_equal(o2, o1 * np.float32(2))


def test_padding_rows_never_read():
    inst = gen.instance_by_name("tiny")
    cfg = inst.cfg
    r = oracle.run_round(inst)
    ids = _concat(inst, "ids")
    w = _concat(inst, "weights")
    used = [set() for _ in range(cfg.F)]
    for f, row in zip(r.layout.slot_part.ravel(), r.layout.slot_row.ravel()):
        if f >= 0:
            used[f].add(int(row))
    poisoned = []
    for f, y in enumerate(r.replies):
        y2 = y.copy()
        pad = [i for i in range(y.shape[0]) if i not in used[f]]
        y2[pad] = 0x7FC0
        y2 = np.concatenate([y2, np.full((5, cfg.H), 0x7FC0, np.uint16)])   # tail rows too
        poisoned.append(y2)
    out = oracle.combine(w, r.layout, cfg.H, poisoned)
    assert np.array_equal(out, r.out)
    assert np.all(np.isfinite(gen.bf16_bits_to_f32(out)))
    assert ids.shape[0] == out.shape[0]


def test_oracle_number_formats():
    import torch
    rng = np.random.default_rng(14)
    v = rng.standard_normal(50000).astype(np.float32)
    ties = (np.arange(500, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties])
    assert np.array_equal(oracle.bf16_round(v),
                          torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])
