"""GPU parity of the per-stage combine (through the C ABI) against the CPU
oracle on the same seeded inputs.

Stage one (each partition's BF16 partial, or its FP8 row of E4M3 codes
and power-of-two scale bytes; design page sections 6 and 19) and stage two
(the float32 sum of the partials in last-lane order, one rounding) are
integer-decided or done in the same float32 operation order on both
sides, so partial rows and outputs must match bit for bit."""
import numpy as np
import pytest

import oracle
from synthetic import gen

pytestmark = pytest.mark.gpu

MODES = ["per_stage", "per_stage_fp8"]


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def check_staged(inst, g, mode):
    from tests.test_gpu_parity import check_round
    cfg = inst.cfg
    ref = oracle.run_round(inst, rows_cap=g.receive_rows, combine_mode=mode)
    mism = check_round(inst, g, ref)
    assert mism == 0, f"{mism} output elements differ from the oracle"
    off = 0
    for s, T in enumerate(cfg.T):
        for f in range(cfg.F):
            has = ref.has[f][off:off + T].astype(bool)
            got = g.partials[s][f]
            if mode == "per_stage":
                want = ref.partial[f][off:off + T].view(np.uint8).reshape(T, 2 * cfg.H)
            else:
                want = ref.qrows[f][off:off + T]
            assert got.shape == want.shape
            bad = np.nonzero((got[has] != want[has]).any(axis=1))[0]
            assert bad.size == 0, f"source {s} partition {f}: {bad.size} partial rows differ"
        off += T


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["tiny", "2a2f_decode", "2a2f_fp8_prefill", "1a3f_e96", "2a2f_skew_h4096"])
def test_staged_parity_workloads(name, mode):
    h = _gpu()
    inst = gen.instance_by_name(name)
    print(f"[staged] {name} {mode}", flush=True)
    g = h.run_round(inst, h.make_buffer(inst, combine=mode))
    check_staged(inst, g, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("i", range(10))
def test_staged_parity_random(i, mode):
    h = _gpu()
    rng = np.random.default_rng(500 + i)
    F = int(rng.integers(2, 5))
    E = F * int(rng.choice([1, 2, 4, 16]))
    K = int(rng.integers(1, min(6, E) + 1))
    N = int(rng.integers(1, 4))
    T = [int(rng.choice([0, 1, 7, 64, 65, 300])) for _ in range(N)]
    if sum(T) == 0:
        T[0] = 9
    H = [256, 512, 768, 1280][i % 4]
    dtype = "fp8" if i % 3 == 2 else "bf16"
    inst = gen.random_small(600 + i, N=N, F=F, E=E, K=K, alpha=int(rng.choice([1, 4, 16])), T=T, H=H,
                            p_skip=0.15, dtype=dtype, bucket=max(T))
    print(f"[staged rand] {i} {mode} T={T} E={E} F={F} K={K} H={H} {dtype}", flush=True)
    g = h.run_round(inst, h.make_buffer(inst, combine=mode), rhc=(i % 2 == 1))
    check_staged(inst, g, mode)


@pytest.mark.parametrize("mode", MODES)
def test_staged_graph_replay_with_inputs_changed(mode):
    """A captured per-stage round replayed with new ids, weights and rows."""
    h = _gpu()
    import torch
    base = dict(N=2, F=3, E=12, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1)
    inst0 = gen.random_small(700, **base)
    cfg = inst0.cfg
    buf = h.make_buffer(inst0, combine=mode)
    dev = h.upload(inst0)
    outs = [torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda") for T in cfg.T]
    h.run_round(inst0, buf, dev, keep_arrays=False, outs=outs)
    torch.cuda.synchronize()
    R = buf.rows_bound(cfg.bucket)
    replies = [torch.empty((R, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.F)]
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        for s, (x, ids, w, sc) in enumerate(dev):
            buf.source_dispatch(s, x, ids, w, sc, bucket=cfg.bucket, out=outs[s])
        recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    with torch.cuda.graph(g2):
        for f in range(cfg.F):
            buf.worker_reply(f, replies[f], recs[f].receipt)
        res = [buf.source_collect(s) for s in range(cfg.N)]
    for rep in range(3):
        inst = gen.random_small(701 + rep, **base)
        for s, src in enumerate(inst.sources):
            dev[s][0].view(torch.int16).copy_(torch.from_numpy(src.x.view(np.int16)))
            dev[s][1].copy_(torch.from_numpy(src.ids))
            dev[s][2].copy_(torch.from_numpy(src.weights))
        g1.replay()
        torch.cuda.synchronize()
        for f in range(cfg.F):
            replies[f].copy_(h.identity_replies(cfg, recs[f], f))
        g2.replay()
        torch.cuda.synchronize()
        ref = oracle.run_round(inst, rows_cap=[R] * cfg.F, combine_mode=mode)
        off = 0
        for s, T in enumerate(cfg.T):
            got = res[s].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, ref.out[off:off + T]), f"replay {rep} source {s}"
            off += T
