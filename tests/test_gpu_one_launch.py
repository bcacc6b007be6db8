"""GPU parity of the one-launch dispatch (AFD_DISPATCH_ONE_LAUNCH, through the
C ABI) against the CPU oracle.

Counts first, then the expansion, in one launch (design page, section 16):
the first 32 workgroups publish per-tile expert counts, a finisher turns
them into every tile's first rows, and the others rank their tokens inside
their tile themselves and wait for those rows.  The
layout must be the same as the split path's: bit-exact ends, rows, scales,
row weights, and the combine to the usual bar.  Also: route errors found by
the counting workgroups, sequences of rounds whose tile counts change (every
launch must read its own counts, never a previous launch's), graph replays,
and the bounded wait's failure path forced from the host (a wait limit
below one poll), which must store nothing, report AFD_E_TIMEOUT and leave
a defined result."""
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


def _buf(h, inst, **kw):
    return h.make_buffer(inst, dispatch="one_launch", **kw)


def _check(inst, g, ref):
    from tests.test_gpu_parity import check_round
    return check_round(inst, g, ref)


@pytest.mark.parametrize("name", ["2a2f_skew_h4096", "2a2f_fp8_prefill", "1a3f_e96", "3a1f_e96_view"])
def test_one_launch_workloads(name):
    h = _gpu()
    inst = gen.instance_by_name(name)
    buf = _buf(h, inst)
    print(f"[one launch] {name}", flush=True)
    g = h.run_round(inst, buf, view=inst.cfg.F == 1)
    assert buf.round_info()["dispatch_path"] == "one_launch"
    assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
    assert buf.get_error(with_status=True)[1] == 0


# (seed, tokens per source, H, K, dtype[, E, F]): tiles of 64, 128 and 256
# tokens, ragged and empty sources, top-k above 8, wide rows, FP8; expert
# counts that are not a multiple of the 32-word table pitch, and up to the
# one-launch limit of 256 experts (the hand-off wavefront then reads four
# experts' words per lane)
CASES = [(0, [600, 0, 41], 512, 8, "bf16"), (1, [1000, 1000], 256, 12, "bf16"), (2, [513], 1024, 4, "fp8"),
         (3, [3000, 2000, 3000], 256, 2, "bf16"), (4, [700], 8448, 8, "bf16"), (5, [2048, 2048], 2048, 32, "fp8"),
         (6, [4096, 4096], 256, 8, "bf16"), (7, [1500, 700], 512, 8, "bf16", 256, 4),
         (8, [900, 37], 512, 6, "fp8", 200, 5)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"c{c[0]}")
def test_one_launch_random(case):
    h = _gpu()
    i, T, H, K, dtype = case[:5]
    F = case[6] if len(case) > 5 else 2 + i % 3
    E = case[5] if len(case) > 5 else (64 if K <= 8 else 128) - (64 if K <= 8 else 128) % F
    inst = gen.random_small(1500 + i, N=len(T), F=F, E=E, K=K, alpha=[1, 16, 128][i % 3],
                            T=T, H=H, p_skip=0.1, dtype=dtype, bucket=max(T))
    buf = _buf(h, inst)
    print(f"[one launch] c{i} T={T} H={H} K={K} {dtype}", flush=True)
    g = h.run_round(inst, buf, rhc=i % 2 == 0)
    assert buf.round_info()["dispatch_path"] == "one_launch"
    assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0


def test_one_launch_rounds_of_changing_tile_counts():
    """Consecutive rounds on one context with 32, 11, 18 and 32 tiles: each
    launch must wait for its own counts, never take a previous launch's."""
    h = _gpu()
    base = gen.random_small(1600, N=2, F=2, E=32, K=8, alpha=8, T=[4096, 4096], H=256, p_skip=0.1, bucket=4096)
    buf = _buf(h, base)
    for j, T in enumerate([[4096, 4096], [600, 50], [1000, 100], [4096, 4000]]):
        inst = gen.generate(dataclasses.replace(base.cfg, T=T, seed=1600 + j))
        print(f"[one launch seq] {T}", flush=True)
        g = h.run_round(inst, buf)
        info = buf.round_info()
        assert info["dispatch_path"] == "one_launch", info
        assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0


def test_one_launch_invalid_routes():
    h = _gpu()
    from tests.test_gpu_rounds import _inject
    inst = _inject(gen.random_small(1700, N=2, F=2, E=16, K=4, alpha=8, T=[700, 900], H=512, p_skip=0.1,
                                    bucket=900), np.random.default_rng(7), n_bad=12)
    cfg = inst.cfg
    err = oracle.layout(cfg.T, np.concatenate([s.ids for s in inst.sources]), cfg.E, cfg.F, cfg.K, cfg.alpha).err
    assert err[0] != 0
    buf = _buf(h, inst)
    g = h.run_round(inst, buf)
    assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
    assert buf.get_error(clear=True) == err
    assert buf.get_error()[0] == 0


def test_one_launch_graph_replays():
    """A captured one-launch round replayed with ids, x and weights changed
    in place (the launch counter lives on the device, so replays tag their
    counts afresh)."""
    from tests import test_gpu_rounds as r
    h = _gpu()
    import harness
    orig = harness.make_buffer
    try:
        harness.make_buffer = lambda inst, **kw: orig(inst, dispatch="one_launch", **kw)
        base = gen.instance_by_name("2a2f_fp8_prefill")
        buf, replay = r._graph_rounds(base)
        for i in range(4):
            inst = gen.generate(dataclasses.replace(base.cfg, seed=base.cfg.seed + 300 + i))
            print(f"[one launch replay] {i}", flush=True)
            g = replay(inst)
            assert buf.round_info()["dispatch_path"] == "one_launch"
            assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
    finally:
        harness.make_buffer = orig
    assert h is not None


def test_one_launch_gives_up_when_told():
    """A wait limit below one poll: every scatter workgroup gives up at once.
    It stores nothing, marks its choices skipped, ends[] is zero and the
    output is +0; afd_get_error reports AFD_E_TIMEOUT until cleared.  The
    next round with the default limit is correct again."""
    h = _gpu()
    import torch
    from combine_layout_amd import _native as nat
    inst = gen.random_small(1800, N=2, F=2, E=32, K=8, alpha=8, T=[700, 300], H=512, p_skip=0.1, bucket=700)
    buf = _buf(h, inst)
    good = h.run_round(inst, buf)
    assert _check(inst, good, oracle.run_round(inst, rows_cap=good.receive_rows)) == 0
    for rows, _, roww in buf.arenas:
        rows.view(torch.int16).fill_(0x1234)
    torch.cuda.synchronize()
    buf.set_dispatch_wait(-1)
    g = h.run_round(inst, buf)
    assert all(np.all(e == 0) for e in g.ends)
    assert all(np.all(o == 0) for o in g.out)
    for rows in g.rows:
        assert np.all(rows == 0x1234)                     # not one row stored
    err, st = buf.get_error(with_status=True)
    assert st == nat.AFD_E_TIMEOUT and err[0] == 0
    assert buf.get_error(clear=True, with_status=True)[1] == nat.AFD_E_TIMEOUT
    assert buf.get_error(with_status=True)[1] == 0
    buf.set_dispatch_wait(1000000)
    g = h.run_round(inst, buf)
    assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
    assert buf.get_error(with_status=True)[1] == 0
