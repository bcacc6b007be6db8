"""Host-side logic of bench.py (CPU only): which kernel the roofline object
names, the median over processes, the 60%-of-peak gate, the time-block
split, and the oracle's OpenMP timing build giving the same bits as the
plain one."""
import numpy as np
import pytest

import bench
import oracle
from synthetic import gen


def test_dominant_kernel_follows_the_reported_path():
    nb = {"dispatch": 10, "combine": 9, "total": 19}
    assert bench.dominant_kernel({"dispatch_path": "one_kernel"}, nb, False, "once") == ("dispatch", "k_fused")
    assert bench.dominant_kernel({"dispatch_path": "tiled"}, nb, False, "once") == ("combine", "k_combine")
    assert bench.dominant_kernel({"dispatch_path": "cached"}, nb, True, "once") == ("dispatch", "k_scatter_cached")
    small = {"dispatch": 5, "combine": 9, "total": 14}
    assert bench.dominant_kernel({"dispatch_path": "one_kernel"}, small, False, "once") == ("combine", "k_combine")
    assert bench.dominant_kernel({"dispatch_path": "tiled"}, nb, False, "per_stage") == \
        ("combine", "k_partial+k_last")


def _fake_run(us, hot, disp, comb):
    return {"workloads": {"2a2f_decode": {
        "us_per_round": us, "us_per_round_blocks": [us], "us_per_round_events": us + 0.6,
        "us_per_round_hot": hot, "bytes_per_round": 18931712,
        "protocol_us_per_round": us - 1.0, "protocol_us_per_round_blocks": [us - 1.0] * 5,
        "protocol_us_per_round_hot": hot - 1.0, "protocol_block_rounds": 256,
        "kernels_us": {"dispatch": disp, "combine": comb}, "identity_experts_us": 50.0, "dispatch_path": "one_kernel",
        "cold_sets": 28, "config": {"workload": "2a2f_decode"}, "inputs_sha256": {},
        "roofline": {"bound": "hbm", "kernel": "k_fused", "achieved": 0.0, "peak": 8000.0, "unit": "GB/s",
                     "frac": 0.0, "traffic": None, "algorithmic_bytes_per_launch": 9478144, "avg_launch_us": disp}}}}


def test_aggregate_takes_medians_and_applies_the_gate():
    class A:
        combine = "once"
        cached = False
        steps = 20
        graph_rounds = 0
    runs = [_fake_run(12.0, 10.0, 6.0, 4.0), _fake_run(10.0, 9.0, 5.0, 4.5), _fake_run(11.0, 11.0, 7.0, 5.0)]
    w = bench.aggregate(runs, ["2a2f_decode"], A)["2a2f_decode"]
    assert w["us_per_round"] == 11.0 and w["us_per_round_hot"] == 10.0
    # the event-timed figure beside the stamped one, and their difference
    # per graph launch (20 rounds in one graph: 0.6 us per round is 12 us)
    assert w["us_per_round_events"] == 11.6 and w["events_minus_stamps_us_per_graph"] == 12.0
    assert w["us_per_round_per_process"] == [12.0, 10.0, 11.0]
    assert w["kernels_us"] == {"dispatch": 6.0, "combine": 4.5}
    assert w["roofline"]["avg_launch_us"] == 6.0
    assert abs(w["roofline"]["frac"] - 9478144 / 6e-6 / 1e9 / 8000) < 1e-4
    # 60% of 8 TB/s for 18,931,712 bytes: 3.944 us; 11 us fails it
    assert w["gate_60pct"] == {"budget_us": 3.944, "pass": False, "pass_protocol": False}
    assert w["protocol"]["us_per_round"] == 10.0 and w["protocol"]["rounds"] == 1280
    assert abs(w["pct_peak"] - 100 * 18931712 / 11e-6 / 1e9 / 8000) < 0.01


def test_oracle_parallel_build_gives_the_same_bits():
    """The all-cores CPU baseline times the same computation."""
    inst = gen.instance_by_name("2a2f_decode")
    cfg = inst.cfg
    ids = np.concatenate([s.ids for s in inst.sources])
    w = np.concatenate([s.weights for s in inst.sources])
    x = np.concatenate([s.x for s in inst.sources])
    ref = oracle.run_round(inst)
    outs = []
    for par in (False, True):
        threads = oracle.set_parallel(par)
        try:
            assert (threads == 1) == (not par)
            lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
            rows, roww = oracle.dispatch(x, w, lay, cfg.F, ref.rows_cap)
            outs.append((rows, roww, oracle.combine(w, lay, cfg.H, ref.replies)))
        finally:
            oracle.set_parallel(False)
    (r0, w0, o0), (r1, w1, o1) = outs
    assert all(np.array_equal(a, b) for a, b in zip(r0, r1))
    assert all(np.array_equal(a, b, equal_nan=True) for a, b in zip(w0, w1))
    assert np.array_equal(o0, o1) and np.array_equal(o0, ref.out)


@pytest.mark.parametrize("name", ["tiny", "2a2f_fp8_prefill"])
def test_cpu_baseline_runs_in_both_settings(name):
    inst = gen.instance_by_name(name)
    for par in (False, True):
        t, n, threads = bench.cpu_baseline(inst, 0.05, par)
        assert t > 0 and n >= 1 and threads >= 1


def test_gated_workloads_are_the_e128_k8_h2048_ones():
    for name in bench.GATED:
        c = gen.instance_by_name(name).cfg
        assert (c.E, c.K, c.H) == (128, 8, 2048)
