"""GPU behaviour beyond one eager round (through the C ABI):

  * graph capture of a round and replays with ids, weights and rows changed
    in place (API contract page, "Graphs, streams and lifetime");
  * invalid routes: sticky first offender and sanitised outputs (design page
    section 8; contract page route rule);
  * determinism against a workspace and arenas poisoned two ways;
  * the single-partition collect view and its copy (design page section 13).
Every result is compared with the CPU oracle on the same inputs."""
import numpy as np
import pytest

import oracle
from synthetic import gen

pytestmark = pytest.mark.gpu


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def _small(seed, **kw):
    base = dict(N=2, F=2, E=16, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1)
    base.update(kw)
    return gen.random_small(seed, **base)


def _check(inst, g, ref):
    from tests.test_gpu_parity import check_round
    return check_round(inst, g, ref)


def test_graph_replay_with_inputs_changed_in_place():
    h = _gpu()
    import torch
    inst0 = _small(1)
    cfg = inst0.cfg
    buf = h.make_buffer(inst0)
    dev = h.upload(inst0)
    outs = [torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda") for T in cfg.T]
    # warm-up round (eager), then capture dispatch+receive and reply+collect
    h.run_round(inst0, buf, dev, keep_arrays=False, outs=outs)
    torch.cuda.synchronize()
    replies = [torch.empty((buf.rows_bound(cfg.bucket), cfg.H), dtype=torch.bfloat16, device="cuda")
               for _ in range(cfg.F)]
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    recs = []
    with torch.cuda.graph(g1):
        for s, (x, ids, w, sc) in enumerate(dev):
            buf.source_dispatch(s, x, ids, w, sc, bucket=cfg.bucket, out=outs[s])
        recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    with torch.cuda.graph(g2):
        for f in range(cfg.F):
            buf.worker_reply(f, replies[f], recs[f].receipt)
        for s in range(cfg.N):
            buf.source_collect(s)
    torch.cuda.synchronize()
    for rep in range(4):
        inst = _small(100 + rep)
        for (x, ids, w, sc), src in zip(dev, inst.sources):
            x.view(torch.int16).copy_(torch.from_numpy(src.x.view(np.int16)))
            ids.copy_(torch.from_numpy(src.ids))
            w.copy_(torch.from_numpy(src.weights))
        if rep == 3:
            for (x, ids, w, sc) in dev:
                ids.fill_(-1)          # every choice inactive
            for src in inst.sources:
                src.ids[:] = -1
        torch.cuda.synchronize()
        g1.replay()
        torch.cuda.synchronize()
        for f, rec in enumerate(recs):
            replies[f].copy_(h.identity_replies(cfg, rec, f))
        g2.replay()
        torch.cuda.synchronize()
        r = h.GpuRound()
        for f, rec in enumerate(recs):
            r.ends.append(rec.ends.cpu().numpy().copy())
            r.host_counts.append(None)
            r.receive_rows.append(rec.receive_rows)
            r.rows.append(rec.rows.view(torch.int16).cpu().numpy().view(np.uint16).copy())
            r.row_weights.append(rec.weights.cpu().numpy().copy())
            r.scales.append(None)
            r.replies.append(replies[f].view(torch.int16).cpu().numpy().view(np.uint16).copy())
        r.out = [o.view(torch.int16).cpu().numpy().view(np.uint16).copy() for o in outs]
        ref = oracle.run_round(inst, rows_cap=r.receive_rows)
        assert _check(inst, r, ref) == 0, f"replay {rep}"
        if rep == 3:
            assert all(np.all(o == 0) for o in r.out)


def _inject(inst, rng, n_bad=6):
    """Plant RANGE, NEG and DUP ids at random places; returns the instance."""
    cfg = inst.cfg
    kinds = [cfg.E + 3, -4, "dup"] * n_bad
    for i in range(n_bad):
        s = int(rng.integers(0, cfg.N))
        if inst.sources[s].ids.shape[0] == 0:
            continue
        t = int(rng.integers(0, inst.sources[s].ids.shape[0]))
        k = int(rng.integers(1, cfg.K))
        kind = kinds[i]
        if kind == "dup":
            inst.sources[s].ids[t, k] = inst.sources[s].ids[t, 0] if inst.sources[s].ids[t, 0] >= 0 else 1
        else:
            inst.sources[s].ids[t, k] = kind
    return inst


# (seed, tokens per source, H): the one-kernel dispatch and the tiled path
# with few and with many tiles
ROUTE_CASES = [(0, [37, 50], 512), (1, [37, 50], 512), (2, [37, 50], 512), (3, [700, 900], 512),
               (4, [5000, 4000], 256)]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"s{c[0]}-{sum(c[1])}")
def test_invalid_routes_sticky_first_offender(case):
    h = _gpu()
    seed, T, H = case
    rng = np.random.default_rng(seed)
    inst = _inject(_small(20 + seed, K=4, T=T, H=H), rng, n_bad=6 if sum(T) < 1000 else 24)
    cfg = inst.cfg
    ids = np.concatenate([s.ids for s in inst.sources])
    lay = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    assert lay.err[0] != 0
    buf = h.make_buffer(inst)
    g = h.run_round(inst, buf)
    ref = oracle.run_round(inst, rows_cap=g.receive_rows)
    assert _check(inst, g, ref) == 0               # outputs are the sanitised result
    code, s, t, k = buf.get_error(clear=False)
    assert (code, s, t, k) == lay.err
    # sticky across a clean round; cleared on request
    clean = _small(40 + seed, T=T, H=H)
    h.run_round(clean, buf)
    assert buf.get_error(clear=True) == lay.err
    assert buf.get_error()[0] == 0


def test_invalid_routes_reported_by_host_count_receive():
    h = _gpu()
    from combine_layout_amd import AfdError
    inst = _inject(_small(60), np.random.default_rng(5))
    buf = h.make_buffer(inst)
    dev = h.upload(inst)
    for s, (x, ids, w, sc) in enumerate(dev):
        buf.source_dispatch(s, x, ids, w, sc, bucket=inst.cfg.bucket, read_host_counts=True)
    with pytest.raises(AfdError):
        buf.worker_receive(0, bucket=inst.cfg.bucket, read_host_counts=True)
    assert buf.get_error(clear=True)[0] != 0


@pytest.mark.parametrize("name", ["2a2f_decode", "1a3f_e96", "2a2f_fp8_prefill"])
def test_deterministic_under_poisoned_workspace(name):
    h = _gpu()
    import torch
    inst = gen.instance_by_name(name)
    results = []
    for fill in (0x00, 0xFF):
        buf = h.make_buffer(inst)
        buf.workspace[256:].fill_(fill)             # keep the error word (first 256 bytes)
        for rows, scales, roww in buf.arenas:
            rows.view(torch.uint8).fill_(fill)
            roww.view(torch.uint8).fill_(fill)
            if scales is not None:
                scales.view(torch.uint8).fill_(fill)
        torch.cuda.synchronize()
        results.append(h.run_round(inst, buf))
    a, b = results
    ref = oracle.run_round(inst, rows_cap=a.receive_rows)
    assert _check(inst, a, ref) == 0 and _check(inst, b, ref) == 0
    for f in range(inst.cfg.F):
        assert np.array_equal(a.ends[f], b.ends[f])
    for s in range(inst.cfg.N):
        assert np.array_equal(a.out[s], b.out[s])


def test_single_partition_view_and_copy():
    h = _gpu()
    import torch
    inst = _small(70, N=3, F=1, E=12, K=4, T=[20, 0, 33])
    cfg = inst.cfg
    buf = h.make_buffer(inst)
    g = h.run_round(inst, buf, view=True)
    ref = oracle.run_round(inst, rows_cap=g.receive_rows)
    assert _check(inst, g, ref) == 0
    views = g.out_tensors
    ws0, ws1 = buf.workspace.data_ptr(), buf.workspace.data_ptr() + buf.workspace.numel()
    for s, v in enumerate(views):
        if cfg.T[s]:
            assert ws0 <= v.data_ptr() < ws1      # aliases the workspace inbox
    # the copy path returns the same values in the caller's output
    g2 = h.run_round(inst, buf, view=False)
    for s in range(cfg.N):
        assert np.array_equal(g2.out[s], g.out[s])
        if cfg.T[s]:
            assert not (ws0 <= g2.out_tensors[s].data_ptr() < ws1)
    # the view lives until the next round's combine rewrites the inbox
    kept = [v.clone() for v in views]
    other = _small(71, N=3, F=1, E=12, K=4, T=[20, 0, 33])
    h.run_round(other, buf, view=True)
    torch.cuda.synchronize()
    assert not torch.equal(views[0], kept[0])
