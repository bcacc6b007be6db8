"""GPU parity of cached dispatch rounds (through the C ABI) against the CPU
oracle.

A cached round (ElasticBuffer page, "Cached Dispatch") reuses the receive
layout of the previous round and scatters new rows, scales and weights
into it.  Its expected result is the oracle's round on the new activations
and weights with the previous round's ids: bit-exact rows, scales, row
weights and ends, and the combine to the same bar as any round."""
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


def _with_ids(new, old):
    """Instance `new` with the expert ids of instance `old` (same shapes)."""
    srcs = [dataclasses.replace(b, ids=a.ids) for a, b in zip(old.sources, new.sources)]
    return gen.Instance(new.cfg, srcs)


def _pair(name_or_inst):
    a = gen.instance_by_name(name_or_inst) if isinstance(name_or_inst, str) else name_or_inst
    b = gen.generate(dataclasses.replace(a.cfg, seed=a.cfg.seed + 1000))
    return a, b


def _check_cached(a, b, combine="once"):
    from tests.test_gpu_parity import check_round
    h = _gpu()
    buf = h.make_buffer(a, combine=combine)
    g1 = h.run_round(a, buf, keep_arrays=False)
    ref_a = oracle.run_round(a, rows_cap=g1.receive_rows,
                             combine_mode=combine)
    assert check_round(a, g1, ref_a, check_rows=False) == 0
    g2 = h.run_round(b, buf, cached=True, view=a.cfg.F == 1)
    hyb = _with_ids(b, a)
    ref = oracle.run_round(hyb, rows_cap=g2.receive_rows, combine_mode=combine)
    assert check_round(hyb, g2, ref) == 0


@pytest.mark.parametrize("name", ["tiny", "2a2f_decode", "2a2f_fp8_prefill", "1a3f_e96", "3a1f_e96_view",
                                  "2a2f_skew_h4096"])
def test_cached_parity_workloads(name):
    a, b = _pair(name)
    print(f"[cached] {name}", flush=True)
    _check_cached(a, b)


@pytest.mark.parametrize("i", range(8))
def test_cached_parity_random(i):
    H = [256, 512, 1024, 4096][i % 4]
    dtype = "fp8" if i % 3 == 1 else "bf16"
    a = gen.random_small(900 + i, H=H, dtype=dtype, T=[[0, 70], [300], [1, 65, 5], [600, 2]][i % 4])
    _, b = _pair(a)
    print(f"[cached rand] {i} T={a.cfg.T} E={a.cfg.E} F={a.cfg.F} K={a.cfg.K} H={H} {dtype}", flush=True)
    _check_cached(a, b)


@pytest.mark.parametrize("mode", ["per_stage", "per_stage_fp8"])
def test_cached_with_per_stage_combine(mode):
    a, b = _pair(gen.random_small(950, N=2, F=3, E=12, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1))
    print(f"[cached {mode}]", flush=True)
    _check_cached(a, b, combine=mode)


def test_cached_graph_replay_with_inputs_changed():
    """A captured cached round replayed with rows and weights changed in place."""
    h = _gpu()
    import torch
    a, _ = _pair(gen.random_small(960, N=2, F=2, E=16, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1))
    cfg = a.cfg
    buf = h.make_buffer(a)
    dev = h.upload(a)
    outs = [torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda") for T in cfg.T]
    h.run_round(a, buf, dev, keep_arrays=False, outs=outs)           # the layout to reuse
    h.run_round(a, buf, dev, keep_arrays=False, outs=outs, cached=True)
    torch.cuda.synchronize()
    R = buf.rows_bound(cfg.bucket)
    replies = [torch.empty((R, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.F)]
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        for s, (x, ids, w, sc) in enumerate(dev):
            buf.source_dispatch(s, x, None, w, sc, bucket=cfg.bucket, out=outs[s], cached=True)
        recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    with torch.cuda.graph(g2):
        for f in range(cfg.F):
            buf.worker_reply(f, replies[f], recs[f].receipt)
        res = [buf.source_collect(s) for s in range(cfg.N)]
    for rep in range(3):
        b = gen.generate(dataclasses.replace(cfg, seed=cfg.seed + 10 + rep))
        for s, src in enumerate(b.sources):
            dev[s][0].view(torch.int16).copy_(torch.from_numpy(src.x.view(np.int16)))
            dev[s][2].copy_(torch.from_numpy(src.weights))
        g1.replay()
        torch.cuda.synchronize()
        for f in range(cfg.F):
            replies[f].copy_(h.identity_replies(cfg, recs[f], f))
        g2.replay()
        torch.cuda.synchronize()
        ref = oracle.run_round(_with_ids(b, a), rows_cap=[R] * cfg.F)
        off = 0
        for s, T in enumerate(cfg.T):
            got = gen.bf16_bits_to_f32(res[s].view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
            want = gen.bf16_bits_to_f32(ref.out[off:off + T]).astype(np.float64)
            assert np.array_equal(got, want), f"replay {rep} source {s}"
            off += T


def test_cached_round_reuses_sanitised_layout():
    """A layout built from ids with invalid routes skips them; a cached round
    reuses that sanitised layout and reports no new offender."""
    h = _gpu()
    from tests.test_gpu_rounds import _inject
    a = _inject(gen.random_small(970, N=2, F=2, E=16, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1),
                np.random.default_rng(3))
    _, b = _pair(a)
    cfg = a.cfg
    lay = oracle.layout(cfg.T, np.concatenate([s.ids for s in a.sources]), cfg.E, cfg.F, cfg.K, cfg.alpha)
    assert lay.err[0] != 0
    buf = h.make_buffer(a)
    h.run_round(a, buf, keep_arrays=False)
    assert buf.get_error(clear=True) == lay.err
    g = h.run_round(b, buf, cached=True)
    hyb = _with_ids(b, a)
    from tests.test_gpu_parity import check_round
    assert check_round(hyb, g, oracle.run_round(hyb, rows_cap=g.receive_rows)) == 0
    assert buf.get_error()[0] == 0
