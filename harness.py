"""GPU-side harness shared by the tests, the smoke check and the benchmark:
uploads a generated instance, runs one round through the library's Python
binding (the C ABI), and plays the FFN with identity experts written in
torch (expert e scales its rows by s_e = 1 + e/E and rounds to bfloat16) --
the stand-in for the caller's expert computation, which is not part of the
library.  It holds none of the exchange's arithmetic and never touches the
CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

from combine_layout_amd import Buffer

NAN_BF16 = 0x7FC0


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def upload(inst):
    """Device tensors for each source: x (bf16 or uint8), ids, weights, scale."""
    out = []
    for src in inst.sources:
        x = to_dev(src.x, torch.bfloat16 if src.x.dtype == np.uint16 else None)
        sc = to_dev(src.scale) if src.scale is not None else None
        out.append((x, to_dev(src.ids), to_dev(src.weights), sc))
    return out


def make_buffer(inst, **kw):
    c = inst.cfg
    return Buffer(c.N, c.F, c.E, c.K, c.H, c.alpha, c.capacity, c.dtype, **kw)


def expert_of_rows(ends: np.ndarray, f: int, E_loc: int, alpha: int, nrows: int) -> np.ndarray:
    """Global expert id of each row of partition f, -1 for padding rows."""
    ex = -np.ones(nrows, np.int64)
    prev = 0
    for j in range(E_loc):
        st = (prev + alpha - 1) // alpha * alpha
        en = int(ends[j])
        ex[st:en] = f * E_loc + j
        prev = en
    return ex


def identity_replies(cfg, rec, f, pad_value=NAN_BF16):
    """Torch identity experts over a received partition; padding rows get
    `pad_value` (NaN by default) so a combine that read them would show."""
    E_loc = cfg.E // cfg.F
    n = rec.receive_rows
    ends = rec.ends.cpu().numpy()
    ex_np = expert_of_rows(ends, f, E_loc, cfg.alpha, n)
    # s_e = 1 + e/E in float32 with a correctly rounded division (numpy);
    # torch's division by a scalar multiplies by the reciprocal instead
    s_np = (np.float32(1.0) + ex_np.astype(np.float32) / np.float32(cfg.E)).astype(np.float32)
    ex = torch.from_numpy(ex_np).cuda()
    s = torch.from_numpy(s_np).cuda()
    if cfg.dtype == "fp8":
        q = rec.rows.view(torch.uint8)[:n].view(torch.float8_e4m3fn).to(torch.float32)
        xv = q * torch.repeat_interleave(rec.scales[:n], 128, dim=1)
    else:
        xv = rec.rows[:n].to(torch.float32)
    y = (xv * s[:, None]).to(torch.bfloat16)
    pad = (ex < 0)
    if pad.any():
        y.view(torch.int16)[pad] = np.int16(np.uint16(pad_value).view(np.int16))
    return y.contiguous()


class GpuRound:
    def __init__(self):
        self.ends = []
        self.host_counts = []
        self.receive_rows = []
        self.rows = []
        self.row_weights = []
        self.scales = []
        self.replies = []
        self.out = []


def run_round(inst, buf=None, dev=None, *, bucket=None, rhc=False, view=False, keep_arrays=True, pad_value=NAN_BF16,
              outs=None, cached=False, reply_order=None):
    """One round through the binding; cached=True dispatches without ids,
    reusing the buffer's last layout; reply_order lists the partitions in
    the order they reply (default ascending)."""
    cfg = inst.cfg
    buf = buf or make_buffer(inst)
    dev = dev or upload(inst)
    bucket = bucket or cfg.bucket
    for s, (x, ids, w, sc) in enumerate(dev):
        o = outs[s] if outs is not None else None
        buf.source_dispatch(s, x, None if cached else ids, w, sc, bucket=bucket, read_host_counts=rhc, out=o,
                            cached=cached)
    recs = [buf.worker_receive(f, bucket=bucket, read_host_counts=rhc) for f in range(cfg.F)]
    replies = [identity_replies(cfg, rec, f, pad_value) for f, rec in enumerate(recs)]
    for f in (range(cfg.F) if reply_order is None else reply_order):
        buf.worker_reply(f, replies[f], recs[f].receipt)
    outs_t = [buf.source_collect(s, view=view) for s in range(cfg.N)]
    torch.cuda.synchronize()
    r = read_round(cfg, recs, replies, outs_t, keep_arrays)
    if buf.combine != "once":
        r.partials = [[buf.partials(s, f).cpu().numpy().copy() for f in range(cfg.F)] for s in range(cfg.N)]
    r.out_tensors = outs_t
    r.buf = buf
    return r


def read_round(cfg, recs, replies, outs, keep_arrays=True):
    """Copy a completed round's receive views, replies and outputs to the
    host (the stream must be synchronised)."""
    r = GpuRound()
    for f, rec in enumerate(recs):
        r.ends.append(rec.ends.cpu().numpy().copy())
        r.host_counts.append(rec.host_counts)
        r.receive_rows.append(rec.receive_rows)
        if keep_arrays:
            if cfg.dtype == "fp8":
                r.rows.append(rec.rows.view(torch.uint8).cpu().numpy().copy())
            else:
                r.rows.append(rec.rows.view(torch.int16).cpu().numpy().view(np.uint16).copy())
            r.row_weights.append(rec.weights.cpu().numpy().copy())
            r.scales.append(rec.scales.cpu().numpy().copy() if rec.scales is not None else None)
            r.replies.append(replies[f].view(torch.int16).cpu().numpy().view(np.uint16).copy())
    r.out = [o.view(torch.int16).cpu().numpy().view(np.uint16).copy() for o in outs]
    return r
