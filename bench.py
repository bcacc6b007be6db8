"""Benchmark of the AFD dispatch+combine round on one MI355X.

A step is one round of the whole hot path for every role: N source
dispatches, F worker receives (layout + scatter), F worker replies (the last
one runs the combine) and N source collects, over one seeded synthetic batch
resident in HBM.  Replies come from identity experts computed once before
timing (expert compute is outside the library and outside the round, as in
the afdEP-comm measurements, which time communication only).

Every workload (the six seeded shapes) is measured by default; the top-level
value is the E128/K8/H2048 decode round the metric names, and a block per
workload carries the same figures.  Rounds are captured in HIP graphs and
replayed.  "cold" rounds rotate over enough independent input/arena/reply
sets to push every round's bytes through HBM past the on-package cache
(round i on set i mod S, so a block's rounds use distinct sets); "hot"
rounds reuse one set.  The timed rounds (--steps after --warmup) run in
graphs of at most 64 rounds, in blocks of at least 64 (one block at 20
steps, since every graph launch has a fixed device-side cost); beside them
the five-block figure runs five blocks of 256 rounds and takes the median
block.  The timed rounds are measured on the GPU's own constant-rate clock,
stamped by tiny kernels captured in the same graph before the first round
and after the last; HIP events around the graph launch are reported beside
them (`us_per_round_events`), since they also hold the graph launch's and
the events' fixed cost (about 12 us per graph here, 0.6 us per round at 20
rounds).  The five-block figure is timed with events (its blocks of 256
rounds spread that cost thin).  Each figure is the median over fresh
processes (three by default).  `value` is the timed rounds' cold
whole-round algorithmic throughput:

  per token       : H*b_x (+4*H/128 FP8 scales) read x, 2*H write the output,
                    8*K read ids+weights, 8*K write + 8*K read the slot map
  per live choice : H*b_x (+ scales) write its row, 2*H read its reply,
                    4 write its row weight

With the CPU baseline (the default), each workload's results are also
compared bit for bit with the oracle's (`parity_vs_oracle`, SHA-256 of the
BF16 outputs).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
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


def partial_rows(inst) -> list:
    """Per partition, the number of tokens with a live choice in it: the
    partial rows that partition's stage one writes."""
    ids = np.concatenate([s.ids for s in inst.sources])
    E_loc = inst.cfg.E // inst.cfg.F
    part = np.where(ids >= 0, ids // E_loc, -1)
    return [int((part == f).any(axis=1).sum()) for f in range(inst.cfg.F)]


def round_bytes(cfg, L: int, combine: str = "once", n_partial=()) -> dict:
    """Algorithmic HBM bytes of one round, split by kernel role.  The
    per-stage combine also writes one partial row per (token, partition)
    with a live choice (BF16, or H codes + scale bytes padded to 32) and
    reads back those of every partition but the last to reply (replies go
    in partition order; the last one's partials are added from registers),
    and each of its F launches reads the slot map."""
    t = byte_terms(cfg, L)
    dispatch = t["x_read"] + t["ids_weights_read"] + t["slot_map_write"] + t["rows_write"] + t["row_weights_write"]
    combine_b = t["replies_read"] + t["slot_map_read"] + t["out_write"]
    if combine != "once":
        prow = 2 * cfg.H if combine == "per_stage" else cfg.H + (cfg.H // 128 + 31) // 32 * 32
        combine_b += (sum(n_partial) + sum(n_partial[:-1])) * prow + (cfg.F - 1) * t["slot_map_read"]
    return {"dispatch": dispatch, "combine": combine_b, "total": dispatch + combine_b}


# ----------------------------------------------------------- GPU harness ----

class RoundSet:
    """One independent set of inputs, outputs, arenas and replies."""

    def __init__(self, inst, view, combine="once", cached=False, dispatch="auto"):
        import torch
        import harness as h
        self.inst = inst
        self.cfg = inst.cfg
        self.view = view
        self.dev = h.upload(inst)
        self.buf = h.make_buffer(inst, combine=combine, dispatch=dispatch)
        self.outs = [torch.empty((T, self.cfg.H), dtype=torch.bfloat16, device="cuda") for T in self.cfg.T]
        # one eager round to obtain the receive layout, then the replies
        for s, (x, ids, w, scl) in enumerate(self.dev):
            self.buf.source_dispatch(s, x, ids, w, scl, bucket=self.cfg.bucket, out=self.outs[s])
        recs = [self.buf.worker_receive(f, bucket=self.cfg.bucket) for f in range(self.cfg.F)]
        self.replies = [h.identity_replies(self.cfg, r, f) for f, r in enumerate(recs)]
        for f, r in enumerate(recs):
            self.buf.worker_reply(f, self.replies[f], r.receipt)
        self.results = [self.buf.source_collect(s, view=view) for s in range(self.cfg.N)]
        torch.cuda.synchronize()
        self.cached = cached

    def output_sha256(self):
        """SHA-256 of the BF16 bits of every source's result in source order
        (after a synchronisation; every round of a set writes the same)."""
        import torch
        h = hashlib.sha256()
        for r in self.results:
            h.update(r.contiguous().view(torch.int16).cpu().numpy().tobytes())
        return h.hexdigest()[:16]

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


class Clock:
    """The GPU's constant-rate real-time counter, stamped by a one-wavefront
    kernel (combine_layout_amd/_lib/libafd_clock.so) that a captured graph
    can hold: timing events cannot be recorded inside a capture, and an
    event pair around a graph launch also measures the launch's fixed cost
    (about 8 us per graph launch and 4 us per event pair here, which at 20
    rounds per graph is 0.6 us per round that no round spends)."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "combine_layout_amd", "_lib", "libafd_clock.so")
        self.lib = ctypes.CDLL(path)
        self.lib.afd_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.afd_clock_hz.argtypes = [ctypes.POINTER(ctypes.c_longlong)]
        hz = ctypes.c_longlong(0)
        if self.lib.afd_clock_hz(ctypes.byref(hz)) != 0:
            raise RuntimeError("afd_clock_hz failed")
        self.hz = float(hz.value)

    def stamp(self, addr):
        """Enqueue a stamp of the counter into the device word at `addr` on
        the current stream."""
        import torch
        if self.lib.afd_clock_stamp(addr, torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("afd_clock_stamp failed")


def capture(sets, order, stamps=None):
    """A graph of one round of each set index in `order`, in that order.
    stamps = (clock, addr0, addr1): the graph also stamps the device clock
    into addr0 before its first round and into addr1 after its last."""
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
        if stamps is not None:
            stamps[0].stamp(stamps[1])
        for i in order:
            sets[i].round()
        if stamps is not None:
            stamps[0].stamp(stamps[2])
    torch.cuda.synchronize()
    return g


class RoundPlan:
    """Graphs for `steps` timed rounds in `blocks` blocks after `warmup`
    untimed ones, rounds numbered from `first`.

    Round i runs on set i mod S, so consecutive rounds use different sets and
    the rounds of a block rotate through distinct ones.  Rounds are replayed
    as graphs of at most `gmax` rounds (cached in `graphs` by starting set
    and length).  Every graph launch has a fixed device-side cost (HIP timing
    events cannot be recorded inside a graph on this runtime), so a block has
    at least 64 rounds: fewer steps make fewer blocks (one, at 20 steps).
    HIP events bracket every block.  With a `clock`, the blocks' graphs are
    captured for this plan alone with a device clock stamp before their
    first round and after their last, and a block's stamped time is the sum
    over its graphs of the stamped spans: the rounds themselves, without the
    graph launches and event records in between (each span also holds the
    first stamp's own short kernel)."""

    def __init__(self, sets, S, first, steps, warmup, graphs, blocks=5, gmax=64, clock=None):
        import torch

        def chunks(start, n, stamped=False):
            out = []
            while n > 0:
                m = min(n, gmax)
                order = [(start + j) % S for j in range(m)]
                if stamped:
                    k = len(self.spans)
                    self.spans.append(k)
                    base = self.stamp_buf.data_ptr() + 16 * k
                    out.append(capture(sets, order, (clock, base, base + 8)))
                else:
                    key = (start % S, m)
                    if key not in graphs:
                        graphs[key] = capture(sets, order)
                    out.append(graphs[key])
                start += m
                n -= m
            return out

        blocks = max(1, min(blocks, steps // 64))
        self.per = [steps // blocks + (1 if b < steps % blocks else 0) for b in range(blocks)]
        self.clock = clock
        self.spans = []
        ngraphs = sum((n + gmax - 1) // gmax for n in self.per)
        self.stamp_buf = torch.zeros((max(1, ngraphs), 2), dtype=torch.int64, device="cuda")
        self.warm = chunks(first, warmup)
        self.blocks = []
        self.block_spans = []
        i = first + warmup
        for n in self.per:
            k0 = len(self.spans)
            self.blocks.append(chunks(i, n, stamped=clock is not None))
            self.block_spans.append(list(range(k0, len(self.spans))))
            i += n
        self.end = i
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]

    def enqueue(self):
        for g in self.warm:
            g.replay()
        self.ev[0].record()
        for b, gs in enumerate(self.blocks):
            for g in gs:
                g.replay()
            self.ev[b + 1].record()

    def result(self):
        """Median block µs per round and every block's value (after a sync),
        from the HIP events."""
        us = [self.ev[b].elapsed_time(self.ev[b + 1]) * 1e3 / n for b, n in enumerate(self.per)]
        return float(np.median(us)), us

    def result_stamped(self):
        """The same from the device clock stamps (plans with a clock)."""
        t = self.stamp_buf.cpu().numpy()
        us = [float(sum(t[k, 1] - t[k, 0] for k in ks)) / self.clock.hz * 1e6 / n
              for ks, n in zip(self.block_spans, self.per)]
        return float(np.median(us)), us


def time_rounds(sets, S, steps, warmup, protocol_steps, protocol_warmup=64, gmax=64, clock=None):
    """The timed steps and the five-block protocol figure on one rotation.

    Every graph is captured first; then the protocol's rounds and, right
    behind them, the `warmup` + `steps` rounds of the timed region are
    enqueued back to back, so the timed steps run on a GPU that has been
    busy for milliseconds (as in a serving loop) rather than one waking from
    the host's capture work, and HIP events between blocks bracket device
    work.  The timed steps' graphs also carry device clock stamps (`clock`).
    Returns ((median, blocks) of the timed steps from the stamps, the same
    from the events, (median, blocks) of the protocol from the events)."""
    import torch
    graphs = {}
    prot = RoundPlan(sets, S, 0, protocol_steps, protocol_warmup, graphs, gmax=gmax)
    timed = RoundPlan(sets, S, prot.end, steps, warmup, graphs, gmax=gmax, clock=clock)
    torch.cuda.synchronize()
    prot.enqueue()
    timed.enqueue()
    torch.cuda.synchronize()
    out = timed.result_stamped(), timed.result(), prot.result()
    del graphs
    return out


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
        for _ in range(2):
            g.replay()                  # untimed, queued ahead: the GPU is busy when t0 is reached
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
    import harness as h
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


def launch_floor(G=32, reps=50):
    """Graph of G rounds of two tiny dependent kernels, replayed `reps` times
    after ten untimed replays queued ahead: the floor a round of two
    launches cannot go below."""
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
    for _ in range(10):
        g.replay()
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (reps * G)


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


def one_way_bandwidth(nbytes, reps=10):
    """A read-only pass (a sum over int32 words) and a write-only pass (a
    fill), each `reps` times over `nbytes`: with the copy, the counter
    calibration's three kernels of known traffic."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    out = []
    for op in (lambda: a.sum(), lambda: b.fill_(7)):
        op()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            op()
        t1.record()
        torch.cuda.synchronize()
        out.append(nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9)
    return out[0], out[1]


# ---------------------------------------------------------- CPU baseline ----

def cpu_baseline(inst, budget_s, parallel=False, ref=None):
    """The oracle as it stands, timed on this host's cores: layout + row,
    scale and weight dispatch + combine per round, the identity-expert
    replies computed once outside the timing (as on the GPU) and every
    output array allocated once before it.  parallel=True runs the oracle's
    OpenMP timing build (row copy and combine on every thread; counting,
    aligned prefix and slots serial).  Returns (seconds per round, rounds,
    threads)."""
    import oracle
    cfg = inst.cfg
    T = cfg.T
    ids = np.concatenate([s.ids for s in inst.sources])
    w = np.concatenate([s.weights for s in inst.sources])
    x = np.concatenate([s.x for s in inst.sources])
    G = cfg.H // 128
    ref = ref or oracle.run_round(inst)
    caps = ref.rows_cap
    threads = oracle.set_parallel(parallel)
    try:
        lay = oracle.layout(T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
        rows = oracle.dispatch(x, w, lay, cfg.F, caps)
        scales = oracle.dispatch_scales(T, [s.scale for s in inst.sources], [(G, 1)] * cfg.N, G, lay, cfg.F,
                                        caps) if cfg.dtype == "fp8" else None
        out = oracle.combine(w, lay, cfg.H, ref.replies)
        rounds = 0
        t_total = 0.0
        while True:
            t0 = time.perf_counter()
            lay = oracle.layout(T, ids, cfg.E, cfg.F, cfg.K, cfg.alpha)
            oracle.dispatch(x, w, lay, cfg.F, caps, out=rows)
            if scales is not None:
                oracle.dispatch_scales(T, [s.scale for s in inst.sources], [(G, 1)] * cfg.N, G, lay, cfg.F, caps,
                                       out=scales)
            oracle.combine(w, lay, cfg.H, ref.replies, out=out)
            t_total += time.perf_counter() - t0
            rounds += 1
            if t_total >= budget_s:
                break
    finally:
        oracle.set_parallel(False)
    return t_total / rounds, rounds, threads


def cpu_model() -> str:
    """The host CPU's model string as lscpu prints it, else /proc/cpuinfo's,
    else the machine type."""
    import subprocess
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            if line.strip().lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
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


# ------------------------------------------------------ GPU measurement ----

# E128 / top-8 / H2048 workloads: the ones the 60%-of-peak target applies to
GATED = ("2a2f_decode", "2a2f_fp8_prefill")
GATE_FRAC = 0.60
MAX_COLD_SETS = 64


def dominant_kernel(info, nb, cached, combine):
    """The single-kernel phase with the most algorithmic bytes, from the
    kernels the library reports for the round: the dispatch when it is one
    kernel (the one-kernel or cached scatter), else the combine; the
    per-stage combine is timed as its whole phase."""
    if combine != "once":
        return "combine", "k_partial+k_last"
    path = info["dispatch_path"]
    single = {"one_kernel": "k_fused", "cached": "k_scatter_cached", "one_launch": "k_dispatch1"}.get(path)
    if single is not None and nb["dispatch"] >= nb["combine"]:
        return "dispatch", single
    return "combine", "k_combine"


def measure_workload(name, args, clock):
    """Every GPU figure of one workload, measured in this process."""
    import torch
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    L = live_choices(inst)
    nb = round_bytes(cfg, L, args.combine, partial_rows(inst) if args.combine != "once" else ())
    view = cfg.F == 1
    S = min(MAX_COLD_SETS, max(1, math.ceil(args.cold_bytes / nb["total"])))
    gmax = args.graph_rounds or 64
    print(f"[bench] {name}: N={cfg.N} T={cfg.T} H={cfg.H} E={cfg.E} F={cfg.F} K={cfg.K} alpha={cfg.alpha} "
          f"dtype={cfg.dtype} L={L} bytes/round={nb['total']} cold sets={S}", file=sys.stderr, flush=True)
    sets = [RoundSet(inst, view, args.combine, args.cached, args.dispatch)]
    info = sets[0].buf.round_info()
    # the five-block protocol beside the timed steps: five blocks of
    # protocol_block rounds after 64 warmup rounds
    (hot_us, hot_blocks), (hot_ev_us, _), (prot_hot_us, _) = time_rounds(
        sets, 1, args.steps, args.warmup, 5 * args.protocol_block, gmax=gmax, clock=clock)
    for _ in range(S - 1):
        sets.append(RoundSet(inst, view, args.combine, args.cached, args.dispatch))
    (cold_us, cold_blocks), (cold_ev_us, cold_ev_blocks), (prot_us, prot_blocks) = time_rounds(
        sets, S, args.steps, args.warmup, 5 * args.protocol_block, gmax=gmax, clock=clock)
    print(f"[bench] {name}: cold {cold_us:.3f} us/round ({args.steps} rounds; events around the graph "
          f"{cold_ev_us:.3f}), hot {hot_us:.3f}; protocol cold {prot_us:.3f} "
          f"(blocks {', '.join(f'{u:.3f}' for u in prot_blocks)}), hot {prot_hot_us:.3f}",
          file=sys.stderr, flush=True)
    kern = time_kernels_live(sets)
    expert_us = time_identity_experts(sets[0])
    dom, dom_name = dominant_kernel(info, nb, args.cached, args.combine)
    mode = ("_cached" if args.cached else "") + ("" if args.combine == "once" else "_" + args.combine) + \
        ("_one_launch" if info["dispatch_path"] == "one_launch" else "")
    traffic = load_traffic(dom_name, name, mode, {"k_partial": cfg.F - 1, "k_last": 1})
    dom_gbps = nb[dom] / (kern[dom] * 1e-6) / 1e9
    gbps = nb["total"] / (cold_us * 1e-6) / 1e9
    res = {
        "us_per_round": cold_us,
        "us_per_round_blocks": cold_blocks,
        "us_per_round_events": cold_ev_us,
        "us_per_round_events_blocks": cold_ev_blocks,
        "us_per_round_hot": hot_us,
        "us_per_round_hot_events": hot_ev_us,
        "us_per_round_hot_blocks": hot_blocks,
        "protocol_us_per_round": prot_us,
        "protocol_us_per_round_blocks": prot_blocks,
        "protocol_us_per_round_hot": prot_hot_us,
        "gbps": gbps,
        "pct_peak": 100 * gbps / PEAK_HBM_GBPS,
        "bytes_per_round": nb["total"],
        "bytes_dispatch": nb["dispatch"],
        "bytes_combine": nb["combine"],
        "kernels_us": kern,
        "identity_experts_us": expert_us,
        "dispatch_path": info["dispatch_path"],
        "layout_tiles": info["layout_tiles"],
        "cold_sets": S,
        "rounds_per_graph_max": gmax,
        "protocol_block_rounds": args.protocol_block,
        "live_choices": L,
        "config": {"workload": name, "sources": cfg.N, "tokens_per_source": cfg.T[0], "hidden": cfg.H,
                   "experts": cfg.E, "partitions": cfg.F, "topk": cfg.K, "expert_alignment": cfg.alpha,
                   "activations": cfg.dtype, "bucket": cfg.bucket, "live_choices": L, "cold_sets": S,
                   "combine": args.combine, "cached_layout": bool(args.cached), "dispatch": args.dispatch},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": dom_gbps, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": dom_gbps / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": nb[dom], "avg_launch_us": kern[dom]},
        "inputs_sha256": inst.digests(),
    }
    torch.cuda.synchronize()
    res["output_sha256"] = sets[0].output_sha256()
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure(names, args):
    """Every selected workload, then the launch floor and the copy rate, in
    this process (which initialises the GPU)."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    clock = Clock()
    out = {"workloads": {}, "clock_hz": clock.hz}
    for name in names:
        out["workloads"][name] = measure_workload(name, args, clock)
    if not args.no_extras:
        out["launch_floor_us_per_round"] = launch_floor()
        out["copy_gbps"] = copy_bandwidth()
    return out


# ------------------------------------------------------------------ main ----

def _median(vals):
    return float(np.median(np.asarray(vals, dtype=np.float64)))


def aggregate(runs, names, args):
    """Per workload, the median over fresh processes of each timing, with
    every process's value kept beside it."""
    out = {}
    for name in names:
        rs = [r["workloads"][name] for r in runs]
        first = rs[0]
        nb = first["bytes_per_round"]
        cold = _median([r["us_per_round"] for r in rs])
        cold_ev = _median([r["us_per_round_events"] for r in rs])
        hot = _median([r["us_per_round_hot"] for r in rs])
        kern = {k: _median([r["kernels_us"][k] for r in rs]) for k in first["kernels_us"]}
        roof = dict(first["roofline"])
        dom = "dispatch" if roof["kernel"] in ("k_fused", "k_scatter_cached", "k_dispatch1") else "combine"
        roof["avg_launch_us"] = kern[dom]
        roof["achieved"] = roof["algorithmic_bytes_per_launch"] / (kern[dom] * 1e-6) / 1e9
        roof["frac"] = roof["achieved"] / PEAK_HBM_GBPS
        gbps = nb / (cold * 1e-6) / 1e9
        prot = _median([r["protocol_us_per_round"] for r in rs])
        prot_hot = _median([r["protocol_us_per_round_hot"] for r in rs])
        w = {
            "us_per_round": round(cold, 3),
            "us_per_round_per_process": [round(r["us_per_round"], 3) for r in rs],
            "us_per_round_blocks": [[round(u, 3) for u in r["us_per_round_blocks"]] for r in rs],
            # the same rounds timed by HIP events around their graph launch:
            # also the launch's and the events' fixed cost, spread over the rounds
            "us_per_round_events": round(cold_ev, 3),
            "us_per_round_events_per_process": [round(r["us_per_round_events"], 3) for r in rs],
            "events_minus_stamps_us_per_graph": round((cold_ev - cold) * args.steps /
                                                      max(1, -(-args.steps // (args.graph_rounds or 64))), 2),
            "gbps": round(gbps, 2),
            "pct_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
            "us_per_round_hot": round(hot, 3),
            "gbps_hot": round(nb / (hot * 1e-6) / 1e9, 2),
            "pct_peak_hot": round(100 * nb / (hot * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
            "protocol": {"us_per_round": round(prot, 3), "pct_peak": round(100 * nb / (prot * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
                         "us_per_round_per_process": [round(r["protocol_us_per_round"], 3) for r in rs],
                         "us_per_round_blocks": [[round(u, 3) for u in r["protocol_us_per_round_blocks"]] for r in rs],
                         "us_per_round_hot": round(prot_hot, 3),
                         "pct_peak_hot": round(100 * nb / (prot_hot * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
                         "rounds": 5 * first["protocol_block_rounds"], "blocks": 5},
            "bytes_per_round": nb,
            "kernels_us": {k: round(v, 3) for k, v in kern.items()},
            "identity_experts_us": round(_median([r["identity_experts_us"] for r in rs]), 3),
            "dispatch_path": first["dispatch_path"],
            "cold_sets": first["cold_sets"],
            "config": first["config"],
            "roofline": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in roof.items()},
            "inputs_sha256": first["inputs_sha256"],
            "output_sha256": [r.get("output_sha256") for r in rs],
        }
        if name in GATED and args.combine == "once" and not args.cached:
            budget = nb / (GATE_FRAC * PEAK_HBM_GBPS * 1e9) * 1e6
            w["gate_60pct"] = {"budget_us": round(budget, 3), "pass": bool(cold <= budget),
                               "pass_protocol": bool(prot <= budget)}
        out[name] = w
    return out


def run_children(args, argv):
    """Measure in `args.processes` fresh processes, one after another; each
    prints its results as one JSON line.  Returns them, or exits with the
    first failing child's status."""
    import subprocess
    runs = []
    child_argv = []
    skip = False
    for a in argv:                           # every argument but --processes (and its value)
        if skip:
            skip = False
        elif a == "--processes":
            skip = True
        elif not a.startswith("--processes="):
            child_argv.append(a)
    for p in range(args.processes):
        print(f"[bench] process {p + 1} of {args.processes}", file=sys.stderr, flush=True)
        proc = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), *child_argv, "--processes", "0",
                               "--child"], stdout=subprocess.PIPE, text=True)
        if proc.returncode != 0:
            print(f"[bench] measuring process {p + 1} failed with status {proc.returncode}", file=sys.stderr)
            sys.exit(proc.returncode if proc.returncode > 0 else 1)
        runs.append(json.loads(proc.stdout.strip().splitlines()[-1]))
    return runs


def main(argv=None):
    argv = list(sys.argv[1:] if argv is None else argv)
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed rounds per workload and process")
    ap.add_argument("--warmup", type=int, default=5, help="untimed rounds before them")
    ap.add_argument("--workload", default="all",
                    help="comma-separated workload names, or 'all' (" + ", ".join(gen.WORKLOADS) + ")")
    ap.add_argument("--headline", default="2a2f_decode", choices=gen.WORKLOADS,
                    help="the workload of the top-level value (the metric's E128/K8/H2048 decode round)")
    ap.add_argument("--processes", type=int, default=3,
                    help="fresh processes to take the median over (0: measure in this process)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--combine", default="once", choices=["once", "per_stage", "per_stage_fp8"],
                    help="combine rounding: once (default), or per stage with BF16 or FP8 partials")
    ap.add_argument("--dispatch", default="auto", choices=["auto", "split", "one_launch"],
                    help="how larger rounds' dispatch is launched (afd_dispatch_mode)")
    ap.add_argument("--cached", action="store_true",
                    help="time rounds that reuse the previous layout (cached dispatch, unchanged routes)")
    ap.add_argument("--graph-rounds", type=int, default=0, help="most rounds per captured graph (default 64)")
    ap.add_argument("--protocol-block", type=int, default=256,
                    help="rounds per block of the five-block protocol figure reported beside the timed steps")
    ap.add_argument("--cold-bytes", type=float, default=512e6, help="bytes the cold rotation spans")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work per setting for the headline workload's CPU baseline")
    ap.add_argument("--cpu-budget-other", type=float, default=1.0,
                    help="seconds per setting for the other workloads' CPU figures")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip launch-floor and copy probes")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read + write), a read-only sum and a "
                         "write-only fill of MIB MiB, ten times each; used to calibrate the HBM byte counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the dispatch/combine path runs every role on a single "
              "device, so there is no multi-GPU configuration to launch (use --gpus 1).", file=sys.stderr)
        return 2
    names = gen.WORKLOADS if args.workload == "all" else args.workload.split(",")
    for n in names:
        if n not in gen.WORKLOADS:
            ap.error(f"unknown workload {n}")
    if args.combine != "once":
        names = [n for n in names if gen.instance_by_name(n).cfg.F >= 2]   # per stage needs two partitions
        if not names:
            ap.error("the per-stage combine needs a workload with two or more partitions")
    headline = args.headline if args.headline in names else names[0]

    if args.copy_only:
        import torch
        torch.cuda.set_device(0)
        gbps = copy_bandwidth(args.copy_only << 20, reps=10)
        read_gbps, write_gbps = one_way_bandwidth(args.copy_only << 20, reps=10)
        print(json.dumps({"copy_mib": args.copy_only, "copy_gbps": round(gbps, 1), "read_gbps": round(read_gbps, 1),
                          "write_gbps": round(write_gbps, 1)}), flush=True)
        return 0
    if args.child or args.processes == 0:
        res = measure(names, args)
        if args.child:
            print(json.dumps(res), flush=True)
            return 0
        runs = [res]
    else:
        runs = run_children(args, argv)     # this process never touches the GPU

    per = aggregate(runs, names, args)
    top = per[headline]
    value = top["gbps"]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(top["us_per_round"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": top["config"],
        "us_per_round": top["us_per_round"],
        "us_per_round_events": top["us_per_round_events"],
        "pct_peak": top["pct_peak"],
        "us_per_round_hot": top["us_per_round_hot"],
        "protocol": top["protocol"],
        "processes": len(runs),
        "roofline": top["roofline"],
    }
    if "gate_60pct" in top:
        line["gate_60pct"] = top["gate_60pct"]
    for k in ("launch_floor_us_per_round", "copy_gbps"):
        if k in runs[0]:
            line[k] = round(_median([r[k] for r in runs]), 3)
    line["workloads"] = per
    if not args.no_cpu:
        import oracle
        model = cpu_model()
        for name in names:
            inst = gen.instance_by_name(name)
            ref = oracle.run_round(inst)
            # the measured rounds' results against the oracle's, bit for bit
            want = oracle.run_round(inst, combine_mode=args.combine) if args.combine != "once" else ref
            want_sha = hashlib.sha256(np.ascontiguousarray(want.out).tobytes()).hexdigest()[:16]
            got = per[name]["output_sha256"]
            per[name]["parity_vs_oracle"] = {"oracle_sha256": want_sha,
                                             "bit_exact": all(g == want_sha for g in got)}
            budget = args.cpu_budget if name == headline else args.cpu_budget_other
            figs = {}
            for par in (False, True):
                t_cpu, n, threads = cpu_baseline(inst, budget, par, ref)
                figs["all_cores" if par else "one_thread"] = (t_cpu, n, threads)
            nb = per[name]["bytes_per_round"]
            per[name]["cpu_oracle"] = {
                k: {"gbps": round(nb / t / 1e9, 4), "ms_per_round": round(t * 1e3, 3), "rounds": n,
                    "threads": th} for k, (t, n, th) in figs.items()}
            if name == headline:
                t, n, th = figs["all_cores"]
                t1, n1, _ = figs["one_thread"]
                line["cpu_baseline"] = {
                    "value": round(nb / t / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
                    "sample": f"{n} full rounds of {name} (layout + dispatch + combine, {t * 1e3:.3f} ms/round; "
                              f"row copy and combine on {th} OpenMP threads, counting and slots serial) on {model}; "
                              f"single-threaded: {n1} rounds, {t1 * 1e3:.3f} ms/round, "
                              f"{nb / t1 / 1e9:.4f} GB/s"}
        line["parity_vs_oracle"] = {"bit_exact": all(per[n]["parity_vs_oracle"]["bit_exact"] for n in names),
                                    "workloads": len(names)}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
