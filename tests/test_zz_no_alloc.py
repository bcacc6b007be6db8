"""The allocation-free context (afd_create_static, through the C ABI) against
the context over a caller workspace (afd_create): two rounds in a row on one
static context, the second smaller, each compared bit for bit with the same
round on an ordinary context (ends, live rows, scales, row weights and the
output), and with the CPU oracle."""
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


def _same(inst, a, b):
    cfg = inst.cfg
    E_loc = cfg.E // cfg.F
    for f in range(cfg.F):
        assert np.array_equal(a.ends[f], b.ends[f]), f"ends of partition {f}"
        prev = 0
        for j in range(E_loc):
            st = (prev + cfg.alpha - 1) // cfg.alpha * cfg.alpha
            en = int(a.ends[f][j])
            assert np.array_equal(a.rows[f][st:en], b.rows[f][st:en])
            assert np.array_equal(a.row_weights[f][st:en], b.row_weights[f][st:en])
            if cfg.dtype == "fp8":
                assert np.array_equal(a.scales[f][st:en], b.scales[f][st:en])
            prev = en
    for s in range(cfg.N):
        assert np.array_equal(a.out[s], b.out[s]), f"output of source {s}"


def _rounds(base, smaller, view=False, dispatch="auto", path=None):
    h = _gpu()
    from combine_layout_amd import AfdError
    from tests.test_gpu_parity import check_round
    c = base.cfg
    ref_buf = h.make_buffer(base, dispatch=dispatch)
    st_buf = h.make_buffer(base, static_workspace=True, dispatch=dispatch)
    try:
        assert st_buf.workspace is None
        with pytest.raises(AfdError):               # one static context per device at a time
            h.make_buffer(base, static_workspace=True)
        for i, inst in enumerate((base, smaller)):
            print(f"[no-alloc] call {i}: T={inst.cfg.T}", flush=True)
            dev = h.upload(inst)
            g_ref = h.run_round(inst, ref_buf, dev, view=view)
            g_st = h.run_round(inst, st_buf, dev, view=view)
            if path is not None:
                assert st_buf.round_info()["dispatch_path"] == path
            _same(inst, g_st, g_ref)
            assert check_round(inst, g_st, oracle.run_round(inst, rows_cap=g_st.receive_rows)) == 0
            if view:
                ws = ref_buf.workspace
                for s, o in enumerate(g_st.out_tensors):
                    if inst.cfg.T[s]:
                        assert not (ws.data_ptr() <= o.data_ptr() < ws.data_ptr() + ws.numel())
    finally:
        st_buf.close()
        ref_buf.close()
    again = h.make_buffer(base, static_workspace=True)   # released by close()
    again.close()
    assert c.N >= 1


def test_static_context_matches_workspace_context():
    """FP8 prefill shape: 2 x 2048 tokens (tiled layout + scatter), then
    2 x (300, 77) tokens (one-kernel dispatch) on the same static scratch."""
    base = gen.instance_by_name("2a2f_fp8_prefill")
    smaller = gen.generate(dataclasses.replace(base.cfg, T=[300, 77], seed=33))
    _rounds(base, smaller)


def test_static_context_single_partition_view():
    """One FFN partition: the collect view points into the static scratch."""
    base = gen.random_small(1400, N=3, F=1, E=12, K=4, alpha=8, T=[600, 0, 333], H=512, p_skip=0.1, bucket=600)
    smaller = gen.generate(dataclasses.replace(base.cfg, T=[20, 5, 0], seed=1401))
    _rounds(base, smaller, view=True)


def test_static_context_one_launch_dispatch():
    """The one-launch dispatch keeps its launch counter and tagged tile
    counts in the workspace, so on the static scratch as well: two tiled
    rounds in a row, the second with fewer tiles."""
    base = gen.instance_by_name("2a2f_skew_h4096")
    smaller = gen.generate(dataclasses.replace(base.cfg, T=[512, 140], seed=34))
    _rounds(base, smaller, dispatch="one_launch", path="one_launch")
