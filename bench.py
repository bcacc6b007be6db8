"""Benchmark of one AFD dispatch+combine round on one MI355X.

A step is one round of the whole hot path for every role: N source
dispatches, F worker receives (layout + scatter), F worker replies (the last
one runs the combine) and N source collects, over one seeded synthetic batch
resident in HBM.  Replies come from identity experts computed once before
timing (expert compute is outside the library and outside the round, as in
the afdEP-comm measurements, which time communication only).

Rounds are captured in HIP graphs and replayed.  "cold" rounds rotate over
enough independent input/arena/reply sets to push every round's bytes through
HBM past the on-package cache; "hot" rounds reuse one set.  `value` is the
cold whole-round algorithmic throughput:

  per token       : H*b_x (+4*H/128 FP8 scales) read x, 2*H write the output,
                    8*K read ids+weights, 8*K write + 8*K read the slot map
  per live choice : H*b_x (+ scales) write its row, 2*H read its reply,
                    4 write its row weight

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synthetic import gen  # noqa: E402

PEAK_HBM_GBPS = 8000.0
METRIC = "dispatch+combine µs/round and achieved HBM GB/s (% peak), E128/K8/H2048"


# ----------------------------------------------------------------- bytes ----

def live_choices(inst) -> int:
    ids = np.concatenate([s.ids for s in inst.sources])
    # generated routes are valid, so every id other than -1 is live
    return int((ids >= 0).sum())


def byte_terms(cfg, L: int) -> dict:
    """Each algorithmic byte stream of one round (ntok tokens, L live choices)."""
    ntok = sum(cfg.T)
    bx = 1 if cfg.dtype == "fp8" else 2
    sc = 4 * (cfg.H // 128) if cfg.dtype == "fp8" else 0
    return {
        "x_read": ntok * (cfg.H * bx + sc),          # source rows (+ scales), read once
        "ids_weights_read": ntok * 8 * cfg.K,         # int32 ids + fp32 weights
        "slot_map_write": ntok * 8 * cfg.K,
        "rows_write": L * (cfg.H * bx + sc),          # expert-major rows (+ scales)
        "row_weights_write": L * 4,
        "replies_read": L * 2 * cfg.H,                # BF16 replies
        "slot_map_read": ntok * 8 * cfg.K,
        "out_write": ntok * 2 * cfg.H,                # BF16 result
    }


def partial_rows(inst) -> int:
    """Number of (token, partition) pairs with a live choice: the partial rows
    a per-stage combine writes and reads."""
    ids = np.concatenate([s.ids for s in inst.sources])
    E_loc = inst.cfg.E // inst.cfg.F
    part = np.where(ids >= 0, ids // E_loc, -1)
    return int(sum((part == f).any(axis=1).sum() for f in range(inst.cfg.F)))


def round_bytes(cfg, L: int, combine: str = "once", n_partial: int = 0) -> dict:
    """Algorithmic HBM bytes of one round, split by kernel role.  The
    per-stage combine also writes and reads one partial row per (token,
    partition) with a live choice (BF16, or H codes + scale bytes padded to
    32), and every partition's stage one reads the slot map."""
    t = byte_terms(cfg, L)
    dispatch = t["x_read"] + t["ids_weights_read"] + t["slot_map_write"] + t["rows_write"] + t["row_weights_write"]
    combine_b = t["replies_read"] + t["slot_map_read"] + t["out_write"]
    if combine != "once":
        prow = 2 * cfg.H if combine == "per_stage" else cfg.H + (cfg.H // 128 + 31) // 32 * 32
        combine_b += 2 * n_partial * prow + cfg.F * t["slot_map_read"]
    return {"dispatch": dispatch, "combine": combine_b, "total": dispatch + combine_b}


# ----------------------------------------------------------- GPU harness ----

class RoundSet:
    """One independent set of inputs, outputs, arenas and replies."""

    def __init__(self, inst, view, combine="once", cached=False):
        import torch
        from tests import gpu_harness as h
        self.inst = inst
        self.cfg = inst.cfg
        self.view = view
        self.dev = h.upload(inst)
        self.buf = h.make_buffer(inst, combine=combine)
        self.outs = [torch.empty((T, self.cfg.H), dtype=torch.bfloat16, device="cuda") for T in self.cfg.T]
        # one eager round to obtain the receive layout, then the replies
        for s, (x, ids, w, scl) in enumerate(self.dev):
            self.buf.source_dispatch(s, x, ids, w, scl, bucket=self.cfg.bucket, out=self.outs[s])
        recs = [self.buf.worker_receive(f, bucket=self.cfg.bucket) for f in range(self.cfg.F)]
        self.replies = [h.identity_replies(self.cfg, r, f) for f, r in enumerate(recs)]
        for f, r in enumerate(recs):
            self.buf.worker_reply(f, self.replies[f], r.receipt)
        for s in range(self.cfg.N):
            self.buf.source_collect(s, view=view)
        torch.cuda.synchronize()
        self.cached = cached

    def dispatch_phase(self):
        """Every source dispatch and worker receive of a round (the receive
        launches the dispatch kernels); returns the receipts.  Cached rounds
        reuse the layout of the set's first round."""
        c = self.cfg
        b = self.buf
        for s, (x, ids, w, scl) in enumerate(self.dev):
            b.source_dispatch(s, x, None if self.cached else ids, w, scl, bucket=c.bucket, out=self.outs[s],
                              cached=self.cached)
        return [b.worker_receive(f, bucket=c.bucket) for f in range(c.F)]

    def combine_phase(self, recs):
        """Every worker reply (the last launches the combine) and source
        collect of a round."""
        c = self.cfg
        b = self.buf
        for f in range(c.F):
            b.worker_reply(f, self.replies[f], recs[f].receipt)
        for s in range(c.N):
            b.source_collect(s, view=self.view)

    def round(self):
        """Enqueue one full round on the current stream."""
        self.combine_phase(self.dispatch_phase())


def capture(sets, order):
    import torch
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in order[:2]:
            sets[i].round()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in order:
            sets[i].round()
    torch.cuda.synchronize()
    return g


def time_graph_rounds(sets, order, steps, warmup, blocks=5):
    """Replay graphs so that exactly `steps` rounds are timed, in `blocks`
    consecutive blocks with an event between blocks; returns the median
    block's µs per round and the per-block values."""
    import torch
    G = len(order)
    g_full = capture(sets, order)
    reps = steps // G
    rem = steps % G
    g_rem = capture(sets, order[:rem]) if rem else None
    for _ in range(max(1, math.ceil(warmup / G))):
        g_full.replay()
    torch.cuda.synchronize()
    blocks = max(1, min(blocks, reps))
    # graph replays per block (the remainder rounds go to the last block)
    per = [reps // blocks + (1 if b < reps % blocks else 0) for b in range(blocks)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for b in range(blocks):
        for _ in range(per[b]):
            g_full.replay()
        if b == blocks - 1 and g_rem is not None:
            g_rem.replay()
        ev[b + 1].record()
    torch.cuda.synchronize()
    us = []
    for b in range(blocks):
        rounds = per[b] * G + (rem if b == blocks - 1 else 0)
        us.append(ev[b].elapsed_time(ev[b + 1]) * 1e3 / rounds)
    return float(np.median(us)), us


def capture_phase(sets, order, phase):
    """One graph holding only the `phase` ("dispatch" or "combine") launches
    of the rounds in `order`.  The other phase of each round is issued on a
    side stream outside the capture, so every round still passes through
    the library in order; inputs are unchanged between rounds, so the
    captured launches read and write what the full rounds do."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for i in order:
            rs = sets[i]
            if phase == "dispatch":
                recs = rs.dispatch_phase()
                with torch.cuda.stream(side):
                    rs.combine_phase(recs)
            else:
                with torch.cuda.stream(side):
                    recs = rs.dispatch_phase()
                rs.combine_phase(recs)
    torch.cuda.synchronize()
    return g


def time_kernels_live(sets, launches=48, reps=8):
    """Average duration of one dispatch and one combine launch, from HIP
    events around replays of graphs that hold `launches` launches of a
    single phase back to back (cycling over the input sets, as the cold
    rounds do), so the events bracket device work only and their own cost
    is spread over many launches."""
    import torch
    order = [i % len(sets) for i in range(launches)]
    out = {}
    for phase in ("dispatch", "combine"):
        g = capture_phase(sets, order, phase)
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        out[phase] = t0.elapsed_time(t1) * 1e3 / (reps * launches)
        del g
    return out


def time_identity_experts(rs, reps=20):
    """Device µs of the identity experts of one round (every partition's
    replies y = bf16(x * s_e) over its rows up to the last aligned live row,
    with the per-row s_e prepared beforehand, as eager torch ops): the
    stand-in for the caller's FFN, outside the round and reported beside
    it."""
    import torch
    from tests import gpu_harness as h
    cfg = rs.cfg
    recs = rs.dispatch_phase()
    rs.combine_phase(recs)
    torch.cuda.synchronize()
    work = []
    for f, r in enumerate(recs):
        # the rows an FFN computes: up to the partition's last aligned live row
        ends = r.ends.cpu().numpy()
        n = int((int(ends[-1]) + cfg.alpha - 1) // cfg.alpha * cfg.alpha) if len(ends) else 0
        ex = h.expert_of_rows(ends, f, cfg.E // cfg.F, cfg.alpha, n)
        s_np = np.where(ex >= 0, np.float32(1.0) + ex.astype(np.float32) / np.float32(cfg.E), np.float32(0.0))
        work.append((r, n, torch.from_numpy(s_np.astype(np.float32)).cuda()))

    def experts():
        for r, n, sc in work:
            if cfg.dtype == "fp8":
                xv = r.rows.view(torch.uint8)[:n].view(torch.float8_e4m3fn).to(torch.float32) * \
                    torch.repeat_interleave(r.scales[:n], 128, dim=1)
            else:
                xv = r.rows[:n].to(torch.float32)
            (xv * sc[:, None]).to(torch.bfloat16)

    experts()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        experts()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps


def launch_floor(G=32, steps=3200):
    """Graph of G rounds of two tiny dependent kernels: the floor a round of
    two launches cannot go below."""
    import torch
    a = torch.zeros(1, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        a.add_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for _ in range(G):
            a.add_(1.0)
            a.mul_(1.0)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps // G):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (steps // G * G)


def copy_bandwidth(nbytes=1 << 30, reps=20):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9


# ---------------------------------------------------------- CPU baseline ----

def cpu_baseline(inst, budget_s=10.0):
    """The oracle as it stands (single-threaded C), timed on this host:
    layout + row/scale/weight dispatch + combine per round, identity-expert
    replies computed once outside the timing (as on the GPU)."""
    import oracle
    cfg = inst.cfg
    T = cfg.T
    ids = np.concatenate([s.ids for s in inst.sources])
    w = np.concatenate([s.weights for s in inst.sources])
    x = np.concatenate([s.x for s in inst.sources])
    G = cfg.H // 128
    ref = oracle.run_round(inst)
    caps = ref.rows_cap
    rounds = 0
    t_total = 0.0
    while True:
        t0 = time.perf_counter()
        lay = oracle.layout(T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
        oracle.dispatch(x, w, lay, cfg.F, caps)
        if cfg.dtype == "fp8":
            oracle.dispatch_scales(T, [s.scale for s in inst.sources], [(G, 1)] * cfg.N, G, lay, cfg.F, caps)
        oracle.combine(w, lay, cfg.H, ref.replies)
        t_total += time.perf_counter() - t0
        rounds += 1
        if t_total >= budget_s:
            break
    return t_total / rounds, rounds


# ------------------------------------------------------------------ main ----

def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def kernel_digest():
    """First 16 hex digits of the SHA-256 of the kernel source's code: the
    text of combine_layout_amd/csrc/afd_kernels.hip with // comments,
    trailing blanks and empty lines removed, so comment edits keep it."""
    import hashlib
    import re
    src = os.path.join(ROOT, "combine_layout_amd", "csrc", "afd_kernels.hip")
    lines = []
    for line in open(src).read().splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def load_traffic(kernel, workload, mode="", mult=None):
    """HBM bytes per dispatch of `kernel` on `workload` (run in `mode`: "" for
    the default round, "_cached" or "_per_stage..." for the others) measured
    with the rocprofv3 counters FETCH_SIZE and WRITE_SIZE (scaled by a
    plain-copy calibration), from the summaries under profiles/ named
    <kernels>_<workload><mode>.md -- None when no summary covers it or the
    kernel source changed since the counters were taken.  A kernel "a+b" is
    the sum of a and b, each times its launches in `mult`."""
    import glob
    digest = kernel_digest()
    parts = kernel.split("+")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}{mode}.md"))):
        text = open(path).read()
        if f"`{digest}`" not in text:
            continue
        for line in text.splitlines():
            line = line.strip()
            if line.startswith("traffic_bytes_per_dispatch "):
                table = json.loads(line[len("traffic_bytes_per_dispatch "):])
                if all(k in table for k in parts):
                    return sum(table[k] * (mult or {}).get(k, 1) for k in parts)
    return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3200)
    ap.add_argument("--warmup", type=int, default=320)
    ap.add_argument("--workload", default="2a2f_decode", choices=gen.WORKLOADS)
    ap.add_argument("--combine", default="once", choices=["once", "per_stage", "per_stage_fp8"],
                    help="combine rounding: once (default), or per stage with BF16 or FP8 partials")
    ap.add_argument("--cached", action="store_true",
                    help="time rounds that reuse the previous layout (cached dispatch, unchanged routes)")
    ap.add_argument("--graph-rounds", type=int, default=0, help="rounds per captured graph (default by size)")
    ap.add_argument("--cold-bytes", type=float, default=512e6, help="bytes the cold rotation spans")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip launch-floor and copy probes")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read + write) ten times; used to "
                         "calibrate the HBM byte counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the dispatch/combine path runs every role on a single "
              "device, so there is no multi-GPU configuration to launch (use --gpus 1).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)

    if args.copy_only:
        gbps = copy_bandwidth(args.copy_only << 20, reps=10)
        print(json.dumps({"copy_mib": args.copy_only, "copy_gbps": round(gbps, 1)}), flush=True)
        return 0

    inst = gen.instance_by_name(args.workload)
    cfg = inst.cfg
    L = live_choices(inst)
    if args.combine != "once" and cfg.F < 2:
        print("the per-stage combine needs two or more partitions", file=sys.stderr)
        return 2
    nb = round_bytes(cfg, L, args.combine, partial_rows(inst) if args.combine != "once" else 0)
    view = cfg.F == 1
    print(f"[bench] {args.workload}: N={cfg.N} T={cfg.T} H={cfg.H} E={cfg.E} F={cfg.F} K={cfg.K} "
          f"alpha={cfg.alpha} dtype={cfg.dtype} L={L} bytes/round={nb['total']}", file=sys.stderr, flush=True)

    S = max(1, math.ceil(args.cold_bytes / nb["total"]))
    G = args.graph_rounds or (32 if nb["total"] < 32e6 else 4)
    G = max(G, S) if S > 1 else G
    G = int(math.ceil(G / S) * S)
    sets = [RoundSet(inst, view, args.combine, args.cached)]
    hot_us, _ = time_graph_rounds(sets, [0] * G, args.steps, args.warmup)
    print(f"[bench] hot: {hot_us:.3f} us/round", file=sys.stderr, flush=True)
    for _ in range(S - 1):
        sets.append(RoundSet(inst, view, args.combine, args.cached))
    cold_us, cold_blocks = time_graph_rounds(sets, [i % S for i in range(G)], args.steps, args.warmup)
    print(f"[bench] cold ({S} sets, {G} rounds/graph): {cold_us:.3f} us/round (median of "
          f"{len(cold_blocks)} blocks: {', '.join(f'{u:.3f}' for u in cold_blocks)})", file=sys.stderr, flush=True)
    expert_us = time_identity_experts(sets[0])

    kern = time_kernels_live(sets)
    # the roofline kernel: the phase with the most algorithmic bytes among
    # those that are one kernel (the combine always; the dispatch when the
    # one-kernel path runs it)
    row_cols = cfg.H * (1 if cfg.dtype == "fp8" else 2) // 16
    fused = sum(cfg.T) <= 512 and sum(cfg.T) * cfg.K <= 4096 and cfg.E <= 256 and row_cols <= 2048
    dom = "dispatch" if fused and nb["dispatch"] >= nb["combine"] else "combine"
    dom_name = {"dispatch": "k_fused", "combine": "k_combine"}[dom]
    if args.cached:
        # the cached dispatch is one kernel at every size
        dom = "dispatch" if nb["dispatch"] >= nb["combine"] else "combine"
        dom_name = {"dispatch": "k_scatter_cached", "combine": "k_combine"}[dom]
    if args.combine != "once":
        # the per-stage combine is F stage-one and N stage-two launches: the
        # phase as a whole
        dom, dom_name = "combine", "k_partial+k_final"
    dom_bytes = nb[dom]
    dom_gbps = dom_bytes / (kern[dom] * 1e-6) / 1e9
    mode = "_cached" if args.cached else ""
    if args.combine != "once":
        mode += "_" + args.combine
    traffic = load_traffic(dom_name, args.workload, mode, {"k_partial": cfg.F, "k_final": cfg.N})

    extras = {}
    if not args.no_extras:
        extras["launch_floor_us_per_round"] = round(launch_floor(), 3)
        extras["copy_gbps"] = round(copy_bandwidth(), 1)

    value = nb["total"] / (cold_us * 1e-6) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "sources": cfg.N, "tokens_per_source": cfg.T[0], "hidden": cfg.H,
                   "experts": cfg.E, "partitions": cfg.F, "topk": cfg.K, "expert_alignment": cfg.alpha,
                   "activations": cfg.dtype, "bucket": cfg.bucket, "live_choices": L, "cold_sets": S,
                   "rounds_per_graph": G, "combine": args.combine, "cached_layout": bool(args.cached)},
        "us_per_round": round(cold_us, 3),
        "us_per_round_blocks": [round(u, 3) for u in cold_blocks],
        "pct_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "us_per_round_hot": round(hot_us, 3),
        "gbps_hot": round(nb["total"] / (hot_us * 1e-6) / 1e9, 2),
        "bytes_per_round": nb["total"],
        "kernels_us": {k: round(v, 3) for k, v in kern.items()},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbps, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(kern[dom], 3)},
    }
    res.update(extras)
    res["identity_experts_us"] = round(expert_us, 3)
    res["inputs_sha256"] = inst.digests()
    if not args.no_cpu:
        t_cpu, n = cpu_baseline(inst, args.cpu_budget)
        res["cpu_baseline"] = {"value": round(nb["total"] / t_cpu / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} full rounds of {args.workload} (layout+dispatch+combine, "
                                         f"{t_cpu * 1e3:.2f} ms/round, single-threaded C oracle, "
                                         f"{cpu_model()})"}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
