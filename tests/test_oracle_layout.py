"""Pins for the oracle's receive layout (CPU only).

The oracle walks choices with per-expert cursors.  These tests re-derive the
layout by different means:
  * the route rule by a per-token set walk;
  * the slots by Python's sorted() over live (expert, source, token) triples,
    placed at a start computed as a sum of aligned counts (not from ends);
  * numpy cumsum (alpha = 1) and a stable numpy argsort (N = F = 1);
and check the invariants the API contract page's ends[] formula implies."""
import itertools

import numpy as np
import pytest

import oracle
from synthetic import gen


def _align(v, a):
    return (v + a - 1) // a * a


def brute_layout(T, ids, E, F, K, alpha):
    E_loc = E // F
    ids = np.asarray(ids).reshape(-1, K)
    live = np.zeros(ids.shape, bool)
    first_err = (0, 0, 0, 0)
    g = 0
    for s, Ts in enumerate(T):
        for t in range(Ts):
            seen = set()
            for k in range(K):
                e = int(ids[g, k])
                code = 0
                if e == -1:
                    pass
                elif e < -1:
                    code = oracle.ROUTE_NEG
                elif e >= E:
                    code = oracle.ROUTE_RANGE
                elif e in seen:
                    code = oracle.ROUTE_DUP
                else:
                    seen.add(e)
                    live[g, k] = True
                if code and first_err[0] == 0:
                    first_err = (code, s, t, k)
            g += 1
    src_of = np.repeat(np.arange(len(T)), T)
    tok_of = np.concatenate([np.arange(Ts) for Ts in T]) if sum(T) else np.zeros(0, int)
    triples = sorted((int(ids[g, k]), int(src_of[g]), int(tok_of[g]), g, k)
                     for g in range(ids.shape[0]) for k in range(K) if live[g, k])
    C = np.zeros(E, np.int64)
    for tr in triples:
        C[tr[0]] += 1
    start = np.zeros(E, np.int64)
    for f in range(F):
        acc = 0
        for j in range(E_loc):
            start[f * E_loc + j] = acc
            acc += _align(int(C[f * E_loc + j]), alpha)
    slot_part = -np.ones(ids.shape, np.int32)
    slot_row = -np.ones(ids.shape, np.int32)
    for e, grp in itertools.groupby(triples, key=lambda tr: tr[0]):
        for rank, tr in enumerate(grp):
            slot_part[tr[3], tr[4]] = e // E_loc
            slot_row[tr[3], tr[4]] = start[e] + rank
    return C, start, slot_part, slot_row, first_err


def _random_ids(rng, ntok, E, K, p_skip=0.2, p_bad=0.0):
    ids = np.argsort(rng.random((ntok, E)), axis=1)[:, :K].astype(np.int32) if ntok else np.zeros((0, K), np.int32)
    ids[rng.random(ids.shape) < p_skip] = -1
    if p_bad:
        bad = rng.random(ids.shape) < p_bad
        kinds = rng.integers(0, 4, ids.shape)
        repl = np.where(kinds == 0, E + rng.integers(0, 5, ids.shape),            # range / "wide"
                        np.where(kinds == 1, -2 - rng.integers(0, 3, ids.shape),  # negative
                                 np.where(kinds == 2, 2 ** 30, ids[:, :1])))     # huge / duplicate of k=0
        ids = np.where(bad, repl, ids).astype(np.int32)
    return ids


SWEEP = []
_r = np.random.default_rng(123)
for _i in range(60):
    F = int(_r.integers(1, 4))
    E = F * int(_r.integers(1, 5))
    K = int(_r.integers(1, min(4, E) + 1))
    N = int(_r.integers(1, 4))
    alpha = int(_r.choice([1, 2, 3, 8]))
    T = [int(_r.choice([0, 1, 5, 64, 65])) for _ in range(N)]
    SWEEP.append((_i, T, E, F, K, alpha))


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"c{c[0]}")
def test_layout_matches_brute_force(case):
    i, T, E, F, K, alpha = case
    rng = np.random.default_rng(i)
    ids = _random_ids(rng, sum(T), E, K, p_skip=0.2, p_bad=0.1 if i % 3 == 0 else 0.0)
    lay = oracle.layout(T, ids, E, F, K, alpha)
    C, start, sp, sr, err = brute_layout(T, ids, E, F, K, alpha)
    assert np.array_equal(lay.slot_part, sp)
    assert np.array_equal(lay.slot_row, sr)
    assert lay.err == err
    assert np.array_equal(lay.ends, (start + C).astype(np.int32))
    assert np.array_equal(lay.host_counts, np.array([_align(int(c), alpha) for c in C], np.int32))
    E_loc = E // F
    for f in range(F):
        assert lay.rows_exact[f] == sum(_align(int(c), alpha) for c in C[f * E_loc:(f + 1) * E_loc])


@pytest.mark.parametrize("case", SWEEP[:30], ids=lambda c: f"c{c[0]}")
def test_layout_invariants(case):
    i, T, E, F, K, alpha = case
    rng = np.random.default_rng(500 + i)
    ids = _random_ids(rng, sum(T), E, K)
    lay = oracle.layout(T, ids, E, F, K, alpha)
    E_loc = E // F
    L = 0
    for f in range(F):
        prev = 0
        targets = set()
        for j in range(E_loc):
            e = f * E_loc + j
            st = _align(prev, alpha)
            assert st % alpha == 0 and 0 <= st - prev < alpha
            C = int(((ids == e) & (lay.slot_part >= 0)).sum())
            assert lay.ends[e] - st == C
            targets.update(range(st, int(lay.ends[e])))
            L += C
            prev = int(lay.ends[e])
        mine = lay.slot_part == f
        rows = lay.slot_row[mine]
        # live choice -> row is a bijection onto the union of expert ranges:
        # every live pair lands exactly once and no padding row is a target
        assert len(set(rows.tolist())) == rows.size
        assert set(rows.tolist()) == targets
    assert L == int((lay.slot_part >= 0).sum())


def test_alpha_one_is_cumsum():
    rng = np.random.default_rng(9)
    T, E, F, K = [40, 33], 12, 3, 3
    ids = _random_ids(rng, sum(T), E, K)
    lay = oracle.layout(T, ids, E, F, K, 1)
    live = lay.slot_part >= 0
    C = np.bincount(ids[live], minlength=E)
    for f in range(F):
        assert np.array_equal(lay.ends[f * 4:(f + 1) * 4], np.cumsum(C[f * 4:(f + 1) * 4]))


def test_single_source_single_partition_is_stable_argsort():
    rng = np.random.default_rng(10)
    T, E, K = [70], 9, 3
    ids = _random_ids(rng, 70, E, K)
    lay = oracle.layout(T, ids, E, 1, K, 1)
    flat = ids.ravel()
    pos = np.flatnonzero(flat >= 0)
    order = pos[np.argsort(flat[pos], kind="stable")]
    expect = -np.ones(flat.size, np.int32)
    expect[order] = np.arange(order.size)
    assert np.array_equal(lay.slot_row.ravel(), expect)


def test_first_offender_codes():
    # one token per error kind, checked in (s, t, k) order
    E, K = 8, 3
    T = [2, 2]
    ids = np.array([[0, 1, 2], [3, 3, 4],      # s0: t1 k1 DUP
                    [9, -5, 1], [2, 2, -7]],   # s1: RANGE at (1,0,0) ...
                   np.int32)
    lay = oracle.layout(T, ids, E, 2, K, 1)
    assert lay.err == (oracle.ROUTE_DUP, 0, 1, 1)
    lay = oracle.layout([2], ids[2:], E, 2, K, 1)
    assert lay.err == (oracle.ROUTE_RANGE, 0, 0, 0)
    lay = oracle.layout([1], np.array([[-1, -2, 8]], np.int32), E, 2, K, 1)
    assert lay.err == (oracle.ROUTE_NEG, 0, 0, 1)
    # a duplicate of a *skipped* choice is live; a duplicate of a live one is not
    lay = oracle.layout([1], np.array([[9, 5, 5]], np.int32), E, 2, K, 1)
    assert lay.err == (oracle.ROUTE_RANGE, 0, 0, 0)
    assert list(lay.slot_part[0]) == [-1, 1, -1]


def test_empty_and_all_skipped():
    lay = oracle.layout([0, 0], np.zeros((0, 2), np.int32), 4, 2, 2, 8)
    assert np.all(lay.ends == 0) and np.all(lay.rows_exact == 0)
    lay = oracle.layout([3], -np.ones((3, 2), np.int32), 4, 2, 2, 8)
    assert np.all(lay.ends == 0) and np.all(lay.slot_part == -1) and lay.err == (0, 0, 0, 0)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_workload_layout_brute_force(name):
    if name in ("2a2f_fp8_prefill", "3a1f_e96_view", "1a3f_e96", "2a2f_skew_h4096"):
        pytest.skip("brute force on the large workloads is covered by the vectorised check below")
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    ids = np.concatenate([s.ids for s in inst.sources])
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    _, _, sp, sr, err = brute_layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    assert np.array_equal(lay.slot_part, sp) and np.array_equal(lay.slot_row, sr) and err == (0, 0, 0, 0)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_workload_layout_vectorised(name):
    """Same check with numpy's stable lexsort standing in for sorted()."""
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    ids = np.concatenate([s.ids for s in inst.sources])
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    g, k = np.nonzero(ids >= 0)              # generator ids are valid: live == not -1
    e = ids[g, k]
    order = np.lexsort((g, e))               # by expert, then global token (= source, token)
    C = np.bincount(e, minlength=cfg.E)
    E_loc = cfg.E // cfg.F
    aligned = (C + cfg.alpha - 1) // cfg.alpha * cfg.alpha
    start = np.zeros(cfg.E, np.int64)
    for f in range(cfg.F):
        a = aligned[f * E_loc:(f + 1) * E_loc]
        start[f * E_loc:(f + 1) * E_loc] = np.concatenate([[0], np.cumsum(a)[:-1]])
    first = np.concatenate([[0], np.cumsum(C)[:-1]])
    rank = np.empty(order.size, np.int64)
    rank[order] = np.arange(order.size) - first[e[order]]
    assert np.array_equal(lay.slot_row[g, k], start[e] + rank)
    assert np.array_equal(lay.slot_part[g, k], e // E_loc)
    assert np.array_equal(lay.ends, (start + C).astype(np.int32))
