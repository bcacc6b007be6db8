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
    import harness
    return harness


def _small(seed, **kw):
    base = dict(N=2, F=2, E=16, K=4, alpha=8, T=[37, 50], H=512, p_skip=0.1)
    base.update(kw)
    return gen.random_small(seed, **base)


def _check(inst, g, ref):
    from tests.test_gpu_parity import check_round
    return check_round(inst, g, ref)


def _graph_rounds(base, view=False):
    """Capture a round of `base`'s shapes as two graphs (dispatch + receive,
    then reply + collect) after an eager warm-up round; returns a function
    that copies an instance of the same shapes into the captured inputs in
    place, replays both graphs (identity-expert replies computed eagerly in
    between) and returns the round read back to the host."""
    h = _gpu()
    import torch
    cfg = base.cfg
    buf = h.make_buffer(base)
    dev = h.upload(base)
    outs = [torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda") for T in cfg.T] if cfg.F > 1 else None
    h.run_round(base, buf, dev, keep_arrays=False, outs=outs, view=view)
    torch.cuda.synchronize()
    replies = [torch.empty((buf.rows_bound(cfg.bucket), cfg.H), dtype=torch.bfloat16, device="cuda")
               for _ in range(cfg.F)]
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        for s, (x, ids, w, sc) in enumerate(dev):
            buf.source_dispatch(s, x, ids, w, sc, bucket=cfg.bucket, out=outs[s] if outs else None)
        recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    with torch.cuda.graph(g2):
        for f in range(cfg.F):
            buf.worker_reply(f, replies[f], recs[f].receipt)
        results = [buf.source_collect(s, view=view) for s in range(cfg.N)]
    torch.cuda.synchronize()

    def replay(inst):
        for (x, ids, w, sc), src in zip(dev, inst.sources):
            if cfg.dtype == "fp8":
                x.copy_(torch.from_numpy(src.x))
                sc.copy_(torch.from_numpy(src.scale))
            else:
                x.view(torch.int16).copy_(torch.from_numpy(src.x.view(np.int16)))
            ids.copy_(torch.from_numpy(src.ids))
            w.copy_(torch.from_numpy(src.weights))
        torch.cuda.synchronize()
        g1.replay()
        torch.cuda.synchronize()
        for f, rec in enumerate(recs):
            replies[f].copy_(h.identity_replies(cfg, rec, f))
        g2.replay()
        torch.cuda.synchronize()
        return h.read_round(cfg, recs, replies, results)

    return buf, replay


# (name, instance): the one-kernel dispatch at a small bucket and at the
# decode workload's bucket of 2048, the tiled layout + scatter at the FP8
# prefill workload, and the single-partition view at the 3A:1F workload
REPLAY_CASES = ["small_one_kernel", "2a2f_decode", "2a2f_fp8_prefill", "3a1f_e96_view"]


def _replay_base(name):
    return _small(1) if name == "small_one_kernel" else gen.instance_by_name(name)


@pytest.mark.parametrize("name", REPLAY_CASES)
def test_graph_replay_with_inputs_changed_in_place(name):
    """API contract page, "Graphs, streams and lifetime": a captured round
    replayed with payloads and ids changed in place, inactive choices as -1.
    Replays: two fresh instances; every choice -1; invalid ids (the
    sanitised result, and the sticky first offender); a clean replay (the
    word stays set: the contract page has invalid routes caught on graph
    replays too); after
    clearing it, a clean replay leaves it clear.  Every replay is compared
    with the oracle on the same inputs."""
    import dataclasses
    base = _replay_base(name)
    cfg = base.cfg
    view = cfg.F == 1
    buf, replay = _graph_rounds(base, view=view)

    def variant(i):
        return gen.generate(dataclasses.replace(cfg, seed=cfg.seed + 100 + i))

    def run(inst, tag):
        print(f"[replay] {name} {tag}", flush=True)
        r = replay(inst)
        ref = oracle.run_round(inst, rows_cap=r.receive_rows)
        assert _check(inst, r, ref) == 0, tag
        return r

    for i in range(2):
        run(variant(i), f"fresh {i}")
        assert buf.get_error()[0] == 0
    skipped = variant(2)
    for src in skipped.sources:
        src.ids[:] = -1
    r = run(skipped, "all -1")
    assert all(np.all(o == 0) for o in r.out)
    assert all(np.all(e == 0) for e in r.ends)
    bad = _inject(variant(3), np.random.default_rng(cfg.seed), n_bad=12)
    ids = np.concatenate([s.ids for s in bad.sources])
    err = oracle.layout(cfg.T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha).err
    assert err[0] != 0
    run(bad, "invalid ids")
    assert buf.get_error() == err
    run(variant(4), "clean after invalid")
    assert buf.get_error(clear=True) == err                 # sticky across replays until cleared
    run(variant(5), "clean after clear")
    assert buf.get_error()[0] == 0


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


def _crafted_ids(ids, E, rng):
    """Overwrite the first rows of a [T, 8] id array with cases aimed at the
    route check's compare-free form (at most eight ids, E <= 248, one byte
    per id, a skip as byte 248 + k): a repeat at each of the 28 position
    pairs, runs of skips, ids at E - 1 and E, ids whose low byte equals an
    id or a skip byte, negatives below -1.  Returns the number of rows set."""
    K = ids.shape[1]

    def distinct():
        return rng.permutation(E)[:K].astype(np.int32)

    rows = []
    for i in range(K):
        for j in range(i + 1, K):
            r = distinct()
            r[j] = r[i]
            rows.append(r)
    for m in range(1, K + 1):                     # m skips at varying places
        r = distinct()
        r[rng.permutation(K)[:m]] = -1
        rows.append(r)
    r = distinct()
    r[3] = E - 1 if E - 1 not in r else r[3]
    rows.append(r)
    for bad in (E, 248, 248 + 5, 256 + int(ids[0, 0] % E), 255, -2, -257, 2 ** 31 - 1, -2 ** 31):
        r = distinct()
        r[5] = bad
        r[2] = -1
        rows.append(r)
    r = distinct()                                 # two skips and a repeat after them
    r[0] = r[1] = -1
    r[7] = r[4]
    rows.append(r)
    n = min(len(rows), ids.shape[0])
    ids[:n] = np.stack(rows[:n])
    return n


# (E, F, tokens, dispatch): E = 248 takes the compare-free check, 249 and 256
# the pairwise one; small rounds run the one-kernel dispatch (above 256
# tokens with two tokens per thread), larger ones the layout kernel, and the
# one-launch dispatch its counting workgroups
ROUTE_BYTES = [(248, 2, 120, "auto"), (249, 3, 120, "auto"), (8, 2, 90, "auto"), (248, 2, 400, "auto"),
               (249, 3, 450, "auto"), (248, 2, 700, "auto"),
               (249, 3, 700, "auto"), (256, 4, 700, "auto"), (248, 4, 700, "one_launch")]


@pytest.mark.parametrize("case", ROUTE_BYTES, ids=lambda c: f"E{c[0]}-T{c[2]}-{c[3]}")
def test_route_check_crafted_ids(case):
    """Both forms of the route check agree with the oracle: the live set of
    every token (so ends, rows, slots and the combine) and the first
    offender of the round."""
    h = _gpu()
    E, F, T, dispatch = case
    rng = np.random.default_rng(E * 7 + T)
    inst = gen.random_small(1300 + E + T, N=1, F=F, E=E, K=8, alpha=4, T=[T], H=256, p_skip=0.0, bucket=T)
    n = _crafted_ids(inst.sources[0].ids, E, rng)
    cfg = inst.cfg
    lay = oracle.layout(cfg.T, inst.sources[0].ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
    assert lay.err[0] != 0 and n > 40
    buf = h.make_buffer(inst, dispatch=dispatch)
    print(f"[route bytes] E={E} T={T} {dispatch}", flush=True)
    g = h.run_round(inst, buf)
    want = {"auto": "one_kernel" if T <= 512 else "tiled", "one_launch": "one_launch"}[dispatch]
    assert buf.round_info()["dispatch_path"] == want
    assert _check(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
    assert buf.get_error(clear=True) == lay.err


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


def test_receive_retried_after_capacity_refusal():
    """Arenas sized for a smaller bucket: the receive is refused with
    AFD_E_CAPACITY and nothing runs; binding arenas for the round's bucket and
    receiving again completes the round, equal to the oracle's."""
    h = _gpu()
    import torch
    from combine_layout_amd import AfdError
    from combine_layout_amd import _native as nat
    inst = _small(80, T=[37, 50], bucket=64)
    cfg = inst.cfg
    buf = h.make_buffer(inst, arena_bucket=8)
    dev = h.upload(inst)
    for s, (x, ids, w, sc) in enumerate(dev):
        buf.source_dispatch(s, x, ids, w, sc, bucket=cfg.bucket)
    with pytest.raises(AfdError) as e:
        buf.worker_receive(0, bucket=cfg.bucket)
    assert e.value.status == nat.AFD_E_CAPACITY
    buf.bind_arenas(cfg.bucket)
    recs = [buf.worker_receive(f, bucket=cfg.bucket) for f in range(cfg.F)]
    replies = [h.identity_replies(cfg, rec, f) for f, rec in enumerate(recs)]
    for f, rec in enumerate(recs):
        buf.worker_reply(f, replies[f], rec.receipt)
    outs = [buf.source_collect(s) for s in range(cfg.N)]
    ref = oracle.run_round(inst, rows_cap=[r.receive_rows for r in recs])
    off = 0
    for s, T in enumerate(cfg.T):
        got = outs[s].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref.out[off:off + T])
        off += T
    # the next round runs on the new arenas
    nxt = _small(81, T=[37, 50], bucket=64)
    g = h.run_round(nxt, buf)
    assert _check(nxt, g, oracle.run_round(nxt, rows_cap=g.receive_rows)) == 0
