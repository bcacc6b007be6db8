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
    import harness
    return harness


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


def _crafted_rows(rng, n, H):
    """BF16 rows whose groups hit every E4M3 rounding case after scaling:
    exact ties between adjacent codes, exact codes, the subnormal range,
    signed zeros, and (one group each) NaN and an infinity."""
    import torch
    pos = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0
    G = H // 128
    out = np.zeros((n, H), np.float32)
    for i in range(n):
        for b in range(G):
            k = int(rng.integers(-100, 100))
            grp = np.concatenate([rng.choice(mids, 60), rng.choice(pos, 40), rng.uniform(-1, 1, 27) * 2.0 ** -8, [448.0]])
            grp = grp * np.where(rng.random(128) < 0.5, -1.0, 1.0)
            grp[5] = 0.0
            grp[6] = -0.0
            rng.shuffle(grp)
            out[i, b * 128:(b + 1) * 128] = (grp * 2.0 ** k).astype(np.float32)
    rows = gen.f32_to_bf16_bits(out)
    rows[0, 3] = 0x7FC0                      # NaN in one group
    if n > 1:
        rows[1, 130] = 0x7F80                # +infinity in another
    return rows


def test_staged_fp8_codes_at_ties_and_specials():
    """K = 1 (weight 1): each partial is its reply row, so crafted replies put
    exact ties, subnormals, signed zeros, NaN and an infinity through the
    kernel's E4M3 encoding, compared byte for byte with the oracle."""
    h = _gpu()
    import torch
    inst = gen.random_small(800, N=2, F=2, E=8, K=1, alpha=4, T=[40, 33], H=512, p_skip=0.0)
    cfg = inst.cfg
    assert np.all(np.concatenate([s.weights for s in inst.sources]) == 1.0)
    buf = h.make_buffer(inst, combine="per_stage_fp8")
    dev = h.upload(inst)
    for s, (x, ids, w, sc) in enumerate(dev):
        buf.source_dispatch(s, x, ids, w, sc, bucket=cfg.bucket)
    recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    rng = np.random.default_rng(801)
    replies_np = [_crafted_rows(rng, r.receive_rows, cfg.H) for r in recs]
    replies = [torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16) for y in replies_np]
    for f, r in enumerate(recs):
        buf.worker_reply(f, replies[f], r.receipt)
    outs = [buf.source_collect(s) for s in range(cfg.N)]
    torch.cuda.synchronize()
    ids = np.concatenate([s.ids for s in inst.sources])
    w = np.concatenate([s.weights for s in inst.sources])
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    partial, has = oracle.combine_partials(w, lay, cfg.H, cfg.F, replies_np)
    q = oracle.quantize_partials(partial, has)
    ref = oracle.combine_stages(lay, cfg.H, None, q)
    off = 0
    for s, T in enumerate(cfg.T):
        for f in range(cfg.F):
            got = buf.partials(s, f).cpu().numpy()
            m = has[f][off:off + T].astype(bool)
            assert np.array_equal(got[m], q[f][off:off + T][m]), f"source {s} partition {f}"
        o = outs[s].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(o, ref[off:off + T]), f"source {s} output"
        off += T


WIDE_F = [(0, 5, 10, 4, [30, 41]), (1, 8, 64, 32, [20, 0, 33]), (2, 16, 32, 12, [70]), (3, 6, 96, 8, [300, 5])]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", WIDE_F, ids=lambda c: f"F{c[1]}K{c[3]}")
def test_staged_parity_many_partitions(case, mode):
    """More than four partitions: stage two requests partials in batches of
    four after reading the slots; top-k up to 32."""
    h = _gpu()
    i, F, E, K, T = case
    inst = gen.random_small(1000 + i, N=len(T), F=F, E=E, K=K, alpha=4, T=T, H=512, p_skip=0.1,
                            dtype="fp8" if i % 2 else "bf16", bucket=max(T))
    print(f"[staged F] F={F} E={E} K={K} T={T} {mode}", flush=True)
    g = h.run_round(inst, h.make_buffer(inst, combine=mode))
    check_staged(inst, g, mode)


# (seed, F, E, K, T, reply order): the last reply is a low or middle
# partition, with at most four partitions and with more
ORDERS = [(0, 2, 16, 8, [300, 41], [1, 0]), (1, 3, 24, 8, [129, 0, 64], [2, 0, 1]),
          (2, 4, 32, 6, [500], [3, 1, 0, 2]), (3, 6, 48, 12, [77, 90], [5, 0, 4, 1, 3, 2]),
          (4, 8, 64, 32, [40, 3], [7, 6, 5, 4, 3, 2, 1, 0])]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ORDERS, ids=lambda c: f"F{c[1]}_last{c[5][-1]}")
def test_staged_reply_order(case, mode):
    """Whichever partition replies last runs its stage one together with
    stage two: partial rows of every partition (the last one's included)
    and outputs equal the oracle's whatever the order."""
    h = _gpu()
    i, F, E, K, T, order = case
    inst = gen.random_small(1200 + i, N=len(T), F=F, E=E, K=K, alpha=8, T=T, H=1024 if i % 2 else 512,
                            p_skip=0.1, dtype="fp8" if i % 2 else "bf16", bucket=max(T))
    print(f"[staged order] F={F} order={order} T={T} {mode}", flush=True)
    g = h.run_round(inst, h.make_buffer(inst, combine=mode), reply_order=order)
    check_staged(inst, g, mode)


@pytest.mark.parametrize("mode", MODES)
def test_staged_with_invalid_routes(mode):
    """Invalid ids are skipped in both stages: partial rows and outputs equal
    the oracle's sanitised result, and the first offender is reported."""
    h = _gpu()
    from tests.test_gpu_rounds import _inject
    inst = _inject(gen.random_small(1100, N=2, F=3, E=12, K=4, alpha=4, T=[37, 50], H=512, p_skip=0.1),
                   np.random.default_rng(11))
    cfg = inst.cfg
    lay = oracle.layout(cfg.T, np.concatenate([s.ids for s in inst.sources]), cfg.E, cfg.F, cfg.K, cfg.alpha)
    assert lay.err[0] != 0
    buf = h.make_buffer(inst, combine=mode)
    g = h.run_round(inst, buf)
    check_staged(inst, g, mode)
    assert buf.get_error(clear=True) == lay.err
