"""GPU parity at the configuration limits and in degenerate rounds (through the
C ABI), against the CPU oracle on the same seeded inputs.

Limits (include/afd.h): 16 sources, 16 partitions, 512 experts, top-32.
Degenerate rounds: every expert chosen by every token (K = E), an
alignment larger than any expert's count, every choice skipped, a single
token.  Wide rows: FP8 rows with more scale blocks than a wavefront has
lanes, and BF16 rows at and past the widest the one-kernel dispatch takes.
Both dispatch paths, both activation formats, and the per-stage and cached
modes are covered."""
import dataclasses

import numpy as np
import pytest

import oracle
from synthetic import gen

pytestmark = pytest.mark.gpu


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness
    return harness


def _run(inst, combine="once", rhc=False):
    from tests.test_gpu_parity import check_round
    h = _gpu()
    g = h.run_round(inst, h.make_buffer(inst, combine=combine), rhc=rhc, view=inst.cfg.F == 1)
    ref = oracle.run_round(inst, rows_cap=g.receive_rows, combine_mode=combine)
    assert check_round(inst, g, ref) == 0
    return g, ref


RAGGED16 = [3, 0, 17, 1, 40, 9, 0, 25, 2, 11, 30, 5, 0, 8, 19, 6]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_limits_tiled_path(dtype):
    """16 ragged sources (some empty), 16 partitions, 512 experts, top-32."""
    inst = gen.random_small(1200, N=16, F=16, E=512, K=32, alpha=128, T=RAGGED16, H=256, p_skip=0.1,
                            dtype=dtype, bucket=64)
    print(f"[limits tiled] {dtype}", flush=True)
    _run(inst, rhc=dtype == "bf16")


def test_limits_one_kernel_path():
    """16 sources x 16 tokens x top-16 = 4096 ids over 256 experts and 16
    partitions: the largest round the one-kernel dispatch takes."""
    inst = gen.random_small(1201, N=16, F=16, E=256, K=16, alpha=16, T=[16] * 16, H=512, p_skip=0.05)
    print("[limits one-kernel]", flush=True)
    _run(inst)


@pytest.mark.parametrize("mode", ["per_stage", "per_stage_fp8"])
def test_limits_per_stage(mode):
    inst = gen.random_small(1202, N=16, F=16, E=512, K=32, alpha=8, T=RAGGED16, H=256, p_skip=0.1, bucket=64)
    print(f"[limits {mode}]", flush=True)
    _run(inst, combine=mode)


def test_limits_cached():
    h = _gpu()
    from tests.test_gpu_parity import check_round
    a = gen.random_small(1203, N=16, F=16, E=512, K=32, alpha=8, T=RAGGED16, H=256, p_skip=0.1, bucket=64)
    b = gen.generate(dataclasses.replace(a.cfg, seed=a.cfg.seed + 1000))
    buf = h.make_buffer(a)
    h.run_round(a, buf, keep_arrays=False)
    g = h.run_round(b, buf, cached=True)
    hyb = gen.Instance(b.cfg, [dataclasses.replace(y, ids=x.ids) for x, y in zip(a.sources, b.sources)])
    assert check_round(hyb, g, oracle.run_round(hyb, rows_cap=g.receive_rows)) == 0


def test_every_expert_chosen():
    """K = E: every token holds every expert (in a random order)."""
    inst = gen.random_small(1204, N=2, F=2, E=8, K=8, alpha=4, T=[33, 70], H=256, p_skip=0.0)
    _run(inst)


def test_alignment_above_every_count():
    """alpha = 1024: every expert's rows start on a 1024 boundary."""
    inst = gen.random_small(1205, N=2, F=2, E=8, K=2, alpha=1024, T=[20, 9], H=256, p_skip=0.2)
    g, ref = _run(inst, rhc=True)
    assert all(int(r) % 1024 == 0 for r in ref.layout.rows_exact)


@pytest.mark.parametrize("F", [1, 2])
def test_every_choice_skipped(F):
    """All ids -1: empty layout, no rows, and +0 outputs (view and copy)."""
    inst = gen.random_small(1206, N=2, F=F, E=8, K=3, alpha=4, T=[10, 7], H=256, p_skip=0.0)
    for s in inst.sources:
        s.ids[:] = -1
    g, ref = _run(inst, rhc=True)
    assert all(int(r) == 0 for r in ref.layout.rows_exact)
    assert all(np.all(o == 0) for o in g.out)


def test_single_token():
    inst = gen.random_small(1207, N=1, F=2, E=4, K=2, alpha=2, T=[1], H=256, p_skip=0.0)
    _run(inst)


WIDE = [("fp8", 16384, [20, 13]),    # one-kernel dispatch, 128 scale blocks per row
        ("fp8", 16384, [600]),       # tiled path: scale blocks past the first 64 take the long-row branch
        ("bf16", 16384, [9, 4]),     # 32 KiB rows: the widest the one-kernel dispatch takes
        ("bf16", 16640, [9, 4])]     # one 16-byte column wider: tiled path even for 13 tokens


@pytest.mark.parametrize("dtype,H,T", WIDE, ids=lambda v: str(v))
def test_wide_rows(dtype, H, T):
    """Rows of 16 K elements and more: FP8 rows carry more scale blocks than a
    wavefront has lanes, and BF16 rows reach and pass the one-kernel limit."""
    inst = gen.random_small(1208, N=len(T), F=2, E=8, K=4, alpha=4, T=T, H=H, p_skip=0.1, dtype=dtype)
    print(f"[limits wide] {dtype} H={H} T={T}", flush=True)
    _run(inst, rhc=dtype == "fp8")


@pytest.mark.parametrize("combine", ["once", "per_stage_fp8"])
def test_wide_fp8_rows_cached(combine):
    """A cached round over FP8 rows with 128 scale blocks (the cached scatter's
    long-row scale branch), and the per-stage FP8 combine over 16 K columns."""
    h = _gpu()
    from tests.test_gpu_parity import check_round
    a = gen.random_small(1209, N=1, F=2, E=8, K=4, alpha=4, T=[600], H=16384, p_skip=0.1, dtype="fp8")
    b = gen.generate(dataclasses.replace(a.cfg, seed=a.cfg.seed + 1000))
    buf = h.make_buffer(a, combine=combine)
    print(f"[limits wide cached] {combine}", flush=True)
    h.run_round(a, buf, keep_arrays=False)
    g = h.run_round(b, buf, cached=True)
    hyb = gen.Instance(b.cfg, [dataclasses.replace(y, ids=x.ids) for x, y in zip(a.sources, b.sources)])
    assert check_round(hyb, g, oracle.run_round(hyb, rows_cap=g.receive_rows, combine_mode=combine)) == 0


EMPTY_OFF_FUSED = [dict(E=512, F=2, K=8, H=256, dtype="bf16"),    # more experts than the one-kernel dispatch takes
                   dict(E=16, F=2, K=4, H=16640, dtype="bf16"),   # rows wider than it takes
                   dict(E=512, F=4, K=4, H=16384, dtype="fp8")]


@pytest.mark.parametrize("kw", EMPTY_OFF_FUSED, ids=lambda d: f"E{d['E']}-H{d['H']}-{d['dtype']}")
def test_all_empty_round_off_the_one_kernel_path(kw):
    """A round in which every source is empty, after a round with tokens on the
    same buffer: ends[] must be all zero again (not the last round's), host
    counts zero and the exact receive size zero, at expert counts and row
    widths the one-kernel dispatch does not take."""
    h = _gpu()
    from tests.test_gpu_parity import check_round
    full = gen.random_small(1210, N=2, alpha=8, T=[30, 700], p_skip=0.1, bucket=700, **kw)
    buf = h.make_buffer(full)
    print(f"[limits empty] {kw}", flush=True)
    g = h.run_round(full, buf, keep_arrays=False)
    assert any(int(e[-1]) > 0 for e in g.ends)
    empty = gen.generate(dataclasses.replace(full.cfg, T=[0, 0]))
    for rhc in (True, False):
        g = h.run_round(empty, buf, rhc=rhc)
        ref = oracle.run_round(empty, rows_cap=g.receive_rows)
        assert check_round(empty, g, ref) == 0
        assert all(np.all(e == 0) for e in g.ends)
        if rhc:
            assert all(r == 0 for r in g.receive_rows)
            assert all(all(c == 0 for c in hc) for hc in g.host_counts)
