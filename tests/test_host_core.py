"""Host core of the C ABI on the CPU (no GPU): argument and configuration
checks, the round state machine, receipts, the workspace plan and the
launch plan.  The core is linked against a recording backend that logs each
device action instead of running it; the HIP library itself is only loaded
to check that it exports every declared symbol."""
import ctypes
import os

import pytest

from combine_layout_amd import _native as nat

FAKE_WS = 1 << 20  # a fake, 256-aligned "device" address; never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nat.FAKE_LIB_PATH):
        from combine_layout_amd import build
        build.build_fake()
    return nat.load_fake()


def log(lib):
    buf = ctypes.create_string_buffer(512)
    out = []
    for i in range(lib.afd_fake_log_size()):
        lib.afd_fake_log_get(i, buf, 512)
        out.append(buf.value.decode())
    lib.afd_fake_log_clear()
    return out


def cfg(N=2, F=2, E=8, K=2, H=256, alpha=4, cap=16, dtype=0, combine=0, dispatch=0):
    return nat.Config(N, F, E, K, H, alpha, cap, dtype, combine, dispatch)


def query(lib, c, bucket):
    ws = ctypes.c_size_t()
    rb = ctypes.c_int64()
    st = lib.afd_query(ctypes.byref(c), bucket, ctypes.byref(ws), ctypes.byref(rb))
    return st, ws.value, rb.value


class Ctx:
    """A created context over fake addresses, with bound arenas."""

    def __init__(self, lib, c, bucket=None, bind=True, cap_rows=None):
        self.lib, self.c = lib, c
        st, ws, rb = query(lib, c, bucket or c.capacity)
        assert st == 0
        self.ws, self.rb = ws, rb
        self.ctx = ctypes.c_void_p()
        assert lib.afd_create(ctypes.byref(c), FAKE_WS, ws, ctypes.byref(self.ctx)) == 0
        if bind:
            for f in range(c.num_partitions):
                sc = 0x300000 + f * 0x1000 if c.dtype == 1 else 0
                assert lib.afd_bind_partition(self.ctx, f, 0x100000 * (f + 4), sc, 0x200000 + f * 0x1000,
                                              cap_rows if cap_rows is not None else rb) == 0

    def dispatch(self, s, T, bucket=None, rhc=0, out=0x7000000, x=0x4000000, ids=0x5000000, w=0x6000000,
                 scale=None, sst=0, ssg=0):
        c = self.c
        if scale is None:
            scale = 0x8000000 if c.dtype == 1 else 0
        return self.lib.afd_source_dispatch(self.ctx, s, T, x if T else 0, ids if T else 0, w if T else 0,
                                            scale if T else 0, sst, ssg, out,
                                            c.capacity if bucket is None else bucket, rhc, None)

    def dispatch_cached(self, s, T, bucket=None, out=0x7000000, x=0x4000000, w=0x6000000, scale=None, sst=0, ssg=0):
        c = self.c
        if scale is None:
            scale = 0x8000000 if c.dtype == 1 else 0
        return self.lib.afd_source_dispatch_cached(self.ctx, s, T, x if T else 0, w if T else 0, scale if T else 0,
                                                   sst, ssg, out, c.capacity if bucket is None else bucket, None)

    def receive(self, f, bucket=None, rhc=0, counts=None):
        rec = nat.Receive()
        hc = (ctypes.c_int32 * (self.c.num_experts // self.c.num_partitions))() if counts else None
        st = self.lib.afd_worker_receive(self.ctx, f, self.c.capacity if bucket is None else bucket, rhc,
                                         ctypes.cast(hc, ctypes.c_void_p) if hc is not None else None,
                                         ctypes.byref(rec), None)
        return st, rec, (list(hc) if hc is not None else None)

    def reply(self, f, rec, rows=None, ptr=0x9000000):
        r = nat.Receipt(rec.receipt.round, rec.receipt.partition, 0)
        return self.lib.afd_worker_reply(self.ctx, f, ptr, rows if rows is not None else rec.receive_rows,
                                         ctypes.byref(r), None)

    def collect(self, s, view=0):
        res = ctypes.c_void_p()
        stride = ctypes.c_int64()
        st = self.lib.afd_source_collect(self.ctx, s, view, ctypes.byref(res), ctypes.byref(stride), None)
        return st, res.value, stride.value

    def full_round(self, T=(4, 3), view=0):
        for s, t in enumerate(T):
            assert self.dispatch(s, t) == 0
        recs = []
        for f in range(self.c.num_partitions):
            st, rec, _ = self.receive(f)
            assert st == 0
            recs.append(rec)
        for f, rec in enumerate(recs):
            assert self.reply(f, rec) == 0
        for s in range(len(T)):
            assert self.collect(s, view)[0] == 0
        return recs

    def destroy(self):
        assert self.lib.afd_destroy(self.ctx) == 0


def test_library_exports_every_declared_symbol():
    syms = nat.header_symbols()
    assert sorted(syms) == sorted(nat.SIGNATURES)        # the binding declares every call
    if not os.path.exists(nat.LIB_PATH):
        pytest.skip("HIP library not built")
    lib = ctypes.CDLL(nat.LIB_PATH)
    for name in syms:
        assert hasattr(lib, name), name
    fake = ctypes.CDLL(nat.FAKE_LIB_PATH)
    for name in syms:
        assert hasattr(fake, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.afd_status_string(st)
    assert lib.afd_status_string(-99) == b"unknown status"


@pytest.mark.parametrize("bad", [
    dict(N=0), dict(N=17), dict(F=0), dict(F=17), dict(E=0), dict(E=513), dict(E=9, F=2),
    dict(K=0), dict(K=33, E=64), dict(K=9, E=8), dict(H=128), dict(H=300), dict(alpha=0), dict(cap=0),
    dict(dtype=2), dict(combine=3), dict(combine=-1), dict(combine=1, F=1, E=4), dict(combine=2, F=1, E=4)])
def test_config_rejected(lib, bad):
    assert query(lib, cfg(**bad), 1)[0] == nat.AFD_E_SHAPE


def test_rows_bound_formula(lib):
    # R_max(bucket) = N * bucket * min(K, E/F) + (E/F) * (alpha - 1)
    for (N, F, E, K, a, b) in [(2, 2, 128, 8, 64, 2048), (1, 3, 96, 8, 128, 2048), (3, 1, 96, 8, 128, 2048),
                               (2, 4, 8, 4, 3, 5), (1, 1, 4, 4, 1, 1)]:
        st, _, rb = query(lib, cfg(N=N, F=F, E=E, K=K, alpha=a, cap=2048), b)
        assert st == 0
        assert rb == N * b * min(K, E // F) + (E // F) * (a - 1)
    assert query(lib, cfg(), 0)[0] == nat.AFD_E_ARG
    assert query(lib, cfg(cap=16), 17)[0] == nat.AFD_E_ARG


def test_rows_must_fit_24_bits(lib):
    # 16 sources x 40000 tokens x 32 choices of one partition: 20.5M rows > 2^24
    assert query(lib, cfg(N=16, F=1, E=64, K=32, cap=40000, alpha=1), 1)[0] == nat.AFD_E_SHAPE
    assert query(lib, cfg(N=16, F=1, E=64, K=32, cap=32000, alpha=1), 1)[0] == 0


def test_workspace_grows_with_capacity_and_inbox(lib):
    _, ws2, _ = query(lib, cfg(F=2, cap=64), 1)
    _, ws1, _ = query(lib, cfg(F=1, cap=64), 1)
    assert ws1 - ws2 >= 2 * 64 * 256 * 2          # the single-partition inboxes
    assert query(lib, cfg(F=2, cap=128), 1)[1] > ws2


def test_create_checks(lib):
    c = cfg()
    _, ws, _ = query(lib, c, 16)
    ctx = ctypes.c_void_p()
    assert lib.afd_create(ctypes.byref(c), 0, ws, ctypes.byref(ctx)) == nat.AFD_E_ARG
    assert lib.afd_create(ctypes.byref(c), FAKE_WS + 8, ws, ctypes.byref(ctx)) == nat.AFD_E_ARG
    assert lib.afd_create(ctypes.byref(c), FAKE_WS, ws - 1, ctypes.byref(ctx)) == nat.AFD_E_CAPACITY
    lib.afd_fake_log_clear()
    assert lib.afd_create(ctypes.byref(c), FAKE_WS, ws, ctypes.byref(ctx)) == 0
    assert log(lib)[0].startswith("init total=")
    assert lib.afd_destroy(ctx) == 0
    assert lib.afd_destroy(None) == 0


def test_bind_checks(lib):
    x = Ctx(lib, cfg(), bind=False)
    L = x.lib
    assert L.afd_bind_partition(x.ctx, 2, 0x100000, 0, 0x200000, 10) == nat.AFD_E_ARG      # index
    assert L.afd_bind_partition(x.ctx, 0, 0x100008, 0, 0x200000, 10) == nat.AFD_E_ARG      # rows alignment
    assert L.afd_bind_partition(x.ctx, 0, 0x100000, 0x300000, 0x200000, 10) == nat.AFD_E_ARG  # scales on BF16
    assert L.afd_bind_partition(x.ctx, 0, 0, 0, 0x200000, 10) == nat.AFD_E_ARG
    assert L.afd_bind_partition(x.ctx, 0, 0x100000, 0, 0x200000, -1) == nat.AFD_E_ARG
    # receive without bound arenas
    assert x.dispatch(0, 2) == 0 and x.dispatch(1, 2) == 0
    assert x.receive(0)[0] == nat.AFD_E_CAPACITY
    x.destroy()
    y = Ctx(lib, cfg(dtype=1), bind=False)
    assert y.lib.afd_bind_partition(y.ctx, 0, 0x100000, 0, 0x200000, 10) == nat.AFD_E_ARG   # FP8 needs scales
    y.destroy()


def test_round_order_and_launch_plan(lib):
    x = Ctx(lib, cfg())
    lib.afd_fake_log_clear()
    # out of order: receive / reply / collect before dispatch
    assert x.receive(0)[0] == nat.AFD_E_ORDER
    assert x.collect(0)[0] == nat.AFD_E_ORDER
    assert x.dispatch(0, 4) == 0
    assert x.dispatch(0, 4) == nat.AFD_E_ORDER                  # twice in one round
    assert x.receive(0)[0] == nat.AFD_E_ORDER                   # source 1 missing
    assert x.dispatch(1, 3, bucket=8) == nat.AFD_E_ARG          # bucket differs in the round
    assert x.dispatch(1, 3, rhc=1) == nat.AFD_E_ARG             # host-count policy differs
    assert x.dispatch(1, 3) == 0
    assert log(lib) == []                                       # dispatch enqueues nothing
    st, r0, _ = x.receive(0)
    assert st == 0
    assert log(lib) == ["dispatch fused=1 ntok=7 nblk=1 T=4,3"]
    assert x.receive(0)[0] == nat.AFD_E_ORDER                   # twice
    st, r1, _ = x.receive(1)
    assert st == 0 and log(lib) == []                           # launched once per round
    assert r0.receive_rows == x.rb and r0.receipt.partition == 0 and r1.receipt.partition == 1
    assert r0.receipt.round == r1.receipt.round == 1
    assert r1.ends - r0.ends == 4 * 4                           # ends of partition 1 follow partition 0's
    assert x.collect(0)[0] == nat.AFD_E_ORDER                   # replies missing
    assert x.reply(0, r1) == nat.AFD_E_ORDER                    # another partition's receipt
    assert x.reply(0, r0, rows=r0.receive_rows - 1) == nat.AFD_E_SHAPE
    assert x.reply(0, r0, ptr=0) == nat.AFD_E_ARG
    assert x.reply(0, r0) == 0
    assert x.reply(0, r0) == nat.AFD_E_ORDER                    # twice
    assert log(lib) == []
    assert x.reply(1, r1) == 0
    assert log(lib) == ["combine ntok=7 out=0x7000000,0x7000000"]
    st, res, stride = x.collect(1)
    assert st == 0 and res == 0x7000000 and stride == 256
    assert x.collect(1)[0] == nat.AFD_E_ORDER
    assert x.collect(0)[0] == 0
    # next round: stale receipt rejected
    x.full_round()
    assert x.dispatch(0, 1) == 0 and x.dispatch(1, 1) == 0
    st, r0b, _ = x.receive(0)
    assert r0b.receipt.round == 3
    assert x.reply(0, r0) == nat.AFD_E_ORDER
    x.destroy()


def test_dispatch_argument_checks(lib):
    x = Ctx(lib, cfg())
    assert x.dispatch(2, 1) == nat.AFD_E_ARG                     # source index
    assert x.dispatch(0, 17, bucket=16) == nat.AFD_E_SHAPE       # T > bucket
    assert x.dispatch(0, 1, bucket=17) == nat.AFD_E_ARG          # bucket > capacity
    assert x.dispatch(0, 1, bucket=0) == nat.AFD_E_ARG
    assert x.dispatch(0, 1, rhc=2) == nat.AFD_E_ARG
    assert x.dispatch(0, 1, x=0x4000008) == nat.AFD_E_ARG        # x not 16-byte aligned
    assert x.dispatch(0, 1, out=0) == nat.AFD_E_ARG              # F > 1 needs out
    assert x.dispatch(0, 1, scale=0x8000000) == nat.AFD_E_ARG    # scales on BF16
    assert x.dispatch(0, -1) == nat.AFD_E_SHAPE
    assert x.dispatch(0, 0, out=0) == 0                          # empty source needs nothing
    x.destroy()
    y = Ctx(lib, cfg(dtype=1))
    assert y.dispatch(0, 2, scale=0) == nat.AFD_E_ARG            # FP8 needs scales
    assert y.dispatch(0, 2, sst=-1) == nat.AFD_E_ARG
    assert y.dispatch(0, 2, sst=1, ssg=2) == 0                   # strided view
    y.destroy()


def test_empty_round_launches_no_combine(lib):
    x = Ctx(lib, cfg())
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 0, out=0) == 0 and x.dispatch(1, 0, out=0) == 0
    recs = [x.receive(f)[1] for f in range(2)]
    assert log(lib) == ["dispatch empty E=8 T=0,0"]
    for f in range(2):
        assert x.reply(f, recs[f]) == 0
    assert log(lib) == []
    assert x.collect(0)[0] == 0 and x.collect(1)[0] == 0
    x.destroy()


@pytest.mark.parametrize("kw", [dict(E=512, F=2, K=8), dict(H=32768), dict(E=512, F=4, K=4, H=16384, dtype=1)],
                         ids=["E512", "H32768", "E512-fp8-H16384"])
def test_empty_round_off_the_one_kernel_path(lib, kw):
    """A round whose sources are all empty clears ends[] at any E and H
    (the one-kernel dispatch covers only E <= 256 and rows of at most 2048
    columns; the tiled path has no tiles to launch)."""
    c = cfg(**kw)
    x = Ctx(lib, c)
    for rnd in range(2):
        lib.afd_fake_log_clear()
        assert x.dispatch(0, 0, out=0) == 0 and x.dispatch(1, 0, out=0) == 0
        recs = [x.receive(f) for f in range(c.num_partitions)]
        assert all(st == 0 for st, _, _ in recs)
        assert log(lib) == [f"dispatch empty E={c.num_experts} T=0,0"]
        for f in range(c.num_partitions):
            assert x.reply(f, recs[f][1]) == 0
        assert log(lib) == []
        assert x.collect(0)[0] == 0 and x.collect(1)[0] == 0
    x.destroy()


def test_receive_retry_after_capacity_failure(lib):
    """A receive refused for a small arena leaves the round open: binding a
    larger arena and receiving again completes it, and the next round runs."""
    c = cfg()
    x = Ctx(lib, c)
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb - 1) == 0
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 2) == 0 and x.dispatch(1, 2) == 0
    assert x.receive(0)[0] == nat.AFD_E_CAPACITY
    assert x.receive(1)[0] == nat.AFD_E_CAPACITY
    assert log(lib) == []                                       # nothing was enqueued
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb) == 0
    recs = []
    for f in range(2):
        st, rec, _ = x.receive(f)
        assert st == 0
        recs.append(rec)
    assert len([l for l in log(lib) if l.startswith("dispatch")]) == 1
    # the dispatch work is enqueued: the arenas are fixed until the round ends
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb) == nat.AFD_E_ORDER
    for f, rec in enumerate(recs):
        assert x.reply(f, rec) == 0
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb) == nat.AFD_E_ORDER
    for s in range(2):
        assert x.collect(s)[0] == 0
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb) == 0   # between rounds
    x.full_round()
    x.destroy()


def test_capacity_check_against_bucket(lib):
    c = cfg()
    x = Ctx(lib, c, cap_rows=None)
    # rebind partition 1 with an arena smaller than R_max(capacity)
    assert lib.afd_bind_partition(x.ctx, 1, 0x100000 * 5, 0, 0x201000, x.rb - 1) == 0
    assert x.dispatch(0, 2) == 0 and x.dispatch(1, 2) == 0
    assert x.receive(0)[0] == nat.AFD_E_CAPACITY
    x.destroy()
    # a smaller bucket needs fewer rows
    y = Ctx(lib, c)
    _, _, rb4 = query(lib, c, 4)
    assert lib.afd_bind_partition(y.ctx, 1, 0x100000 * 5, 0, 0x201000, rb4) == 0
    for s in range(2):
        assert y.dispatch(s, 3, bucket=4) == 0
    st, rec, _ = y.receive(1, bucket=4)
    assert st == 0 and rec.receive_rows == rb4
    y.destroy()


def test_read_host_counts(lib):
    c = cfg(E=8, F=2, alpha=4)
    x = Ctx(lib, c)
    ends = (ctypes.c_int32 * 8)(3, 8, 8, 9, 1, 7, 9, 12)      # partition 0: C = 3,4,0,1; partition 1: 1,3,1,0
    lib.afd_fake_set_ends(ctypes.cast(ends, ctypes.c_void_p), 8, nat_err_none())
    lib.afd_fake_log_clear()
    for s in range(2):
        assert x.dispatch(s, 4, rhc=1) == 0
    st, r0, hc0 = x.receive(0, rhc=1, counts=True)
    assert st == 0
    assert log(lib) == ["dispatch fused=1 ntok=8 nblk=1 T=4,4", "read_ends E=8"]
    assert hc0 == [4, 4, 0, 4] and r0.receive_rows == 12
    st, r1, hc1 = x.receive(1, rhc=1, counts=True)
    assert st == 0 and log(lib) == []
    assert hc1 == [4, 4, 4, 0] and r1.receive_rows == 12
    assert x.receive(0)[0] == nat.AFD_E_ORDER
    x.destroy()
    # host counts requested without read_host_counts
    y = Ctx(lib, c)
    for s in range(2):
        assert y.dispatch(s, 4) == 0
    assert y.receive(0, counts=True)[0] == nat.AFD_E_ARG
    y.destroy()


def nat_err_none():
    return ctypes.c_uint64(0xFFFFFFFFFFFFFFFF).value


def test_read_host_counts_refused_while_capturing(lib):
    x = Ctx(lib, cfg())
    for s in range(2):
        assert x.dispatch(s, 2, rhc=1) == 0
    lib.afd_fake_set_capturing(1)
    try:
        assert x.receive(0, rhc=1)[0] == nat.AFD_E_ARG
    finally:
        lib.afd_fake_set_capturing(0)
    assert x.receive(0, rhc=1)[0] == 0
    x.destroy()


def test_route_error_word_decoding(lib):
    x = Ctx(lib, cfg())
    word = (3 << 56) | (1234 << 24) | (7 << 16) | 2       # source 3, token 1234, k 7, NEG
    ends = (ctypes.c_int32 * 8)()
    lib.afd_fake_set_ends(ctypes.cast(ends, ctypes.c_void_p), 8, word)
    code, s, t, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib.afd_get_error(x.ctx, None, 0, ctypes.byref(code), ctypes.byref(s), ctypes.byref(t), ctypes.byref(k))
    assert st == nat.AFD_E_ROUTE and (code.value, s.value, t.value, k.value) == (2, 3, 1234, 7)
    # a receive with host counts reports it too, after completing the round's layout
    for q in range(2):
        assert x.dispatch(q, 2, rhc=1) == 0
    st, rec, _ = x.receive(0, rhc=1)
    assert st == nat.AFD_E_ROUTE and rec.receipt.round == 1
    assert x.receive(0, rhc=1)[0] == nat.AFD_E_ORDER           # the receive did complete
    st = lib.afd_get_error(x.ctx, None, 1, ctypes.byref(code), None, None, None)
    assert st == nat.AFD_E_ROUTE
    st = lib.afd_get_error(x.ctx, None, 0, ctypes.byref(code), ctypes.byref(s), None, None)
    assert st == 0 and code.value == 0 and s.value == -1
    lib.afd_fake_set_capturing(1)
    try:
        assert lib.afd_get_error(x.ctx, None, 0, None, None, None, None) == nat.AFD_E_ARG
    finally:
        lib.afd_fake_set_capturing(0)
    x.destroy()


def test_single_partition_view_and_copy(lib):
    c = cfg(F=1, E=4, N=2)
    x = Ctx(lib, c)
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 3, out=0x7000000) == 0
    assert x.dispatch(1, 2, out=0) == 0                          # out optional with one partition
    st, rec, _ = x.receive(0)
    assert x.reply(0, rec) == 0
    lg = log(lib)
    inbox0 = int(lg[1].split("out=")[1].split(",")[0], 16)
    inbox1 = int(lg[1].split("out=")[1].split(",")[1], 16)
    assert inbox1 - inbox0 == c.capacity * c.hidden * 2          # one inbox per source in the workspace
    assert FAKE_WS < inbox0 < FAKE_WS + x.ws
    st, res, stride = x.collect(1, view=0)
    assert st == nat.AFD_E_ARG                                   # no out for a copy
    st, res, stride = x.collect(1, view=1)
    assert st == 0 and res == inbox1 and stride == c.hidden
    st, res, _ = x.collect(0, view=0)
    assert st == 0 and res == 0x7000000
    assert log(lib) == [f"copy {hex(inbox0)}->0x7000000 bytes={3 * 256 * 2}"]
    x.destroy()


def test_split_path_above_fused_limits(lib):
    # above 512 tokens: tiled layout (the smallest of 64/128/256-token tiles
    # that keeps a round within 32 tiles)
    c = cfg(N=2, F=2, E=8, K=2, cap=2048)
    x = Ctx(lib, c)
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 300) == 0 and x.dispatch(1, 1000) == 0
    assert x.receive(0)[0] == 0
    assert log(lib) == ["dispatch fused=0 ntok=1300 nblk=21 T=300,1000 tile=64 voff=0,320,1344"]
    x.destroy()
    # more than 4096 ids
    y = Ctx(lib, cfg(N=1, F=2, E=32, K=16, cap=2048))
    lib.afd_fake_log_clear()
    assert y.dispatch(0, 300) == 0
    assert y.receive(0)[0] == 0
    assert log(lib) == ["dispatch fused=0 ntok=300 nblk=5 T=300 tile=64 voff=0,320"]
    y.destroy()
    # more than 256 experts
    z = Ctx(lib, cfg(N=1, F=2, E=512, K=4, cap=2048))
    lib.afd_fake_log_clear()
    assert z.dispatch(0, 600) == 0
    assert z.receive(0)[0] == 0
    assert log(lib) == ["dispatch fused=0 ntok=600 nblk=10 T=600 tile=64 voff=0,640"]
    z.destroy()
    # many tiles and 16 KB rows
    u = Ctx(lib, cfg(N=2, F=2, E=8, K=2, cap=8192))
    lib.afd_fake_log_clear()
    assert u.dispatch(0, 5000) == 0 and u.dispatch(1, 4000) == 0
    assert u.receive(0)[0] == 0
    assert log(lib) == ["dispatch fused=0 ntok=9000 nblk=36 T=5000,4000 tile=256 voff=0,5120,9216"]
    u.destroy()
    v = Ctx(lib, cfg(N=1, F=2, E=8, K=2, H=8192, cap=2048))
    lib.afd_fake_log_clear()
    assert v.dispatch(0, 600) == 0
    assert v.receive(0)[0] == 0
    assert log(lib) == ["dispatch fused=0 ntok=600 nblk=10 T=600 tile=64 voff=0,640"]
    v.destroy()


def test_split_path_sources_start_on_tile_boundaries(lib):
    # every source starts on a tile boundary of the tiled token space, empty
    # sources take no space, and the tile grows until the round fits 32 tiles
    x = Ctx(lib, cfg(N=3, F=2, E=8, K=2, cap=4096))
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 65) == 0 and x.dispatch(1, 0) == 0 and x.dispatch(2, 500) == 0
    assert x.receive(0)[0] == 0
    # 65 -> two 64-slot tiles, 0 -> none, 500 -> eight: 10 tiles (9 without the padding)
    assert log(lib) == ["dispatch fused=0 ntok=565 nblk=10 T=65,0,500 tile=64 voff=0,128,128,640"]
    x.destroy()
    y = Ctx(lib, cfg(N=3, F=2, E=8, K=2, cap=4096))
    lib.afd_fake_log_clear()
    assert y.dispatch(0, 1) == 0 and y.dispatch(1, 2100) == 0 and y.dispatch(2, 1) == 0
    assert y.receive(0)[0] == 0
    # 64-slot tiles would need 1 + 33 + 1 = 35 tiles; 128-slot tiles: 1 + 17 + 1 = 19
    assert log(lib) == ["dispatch fused=0 ntok=2102 nblk=19 T=1,2100,1 tile=128 voff=0,128,2304,2432"]
    y.destroy()


def tiles(lib):
    buf = (ctypes.c_int32 * (4 * 32))()
    n = lib.afd_fake_tiles(ctypes.cast(buf, ctypes.c_void_p), 32)
    return [tuple(buf[4 * b:4 * b + 4]) for b in range(n)]


def test_layout_tile_records(lib):
    # each layout tile's record: (source, first token in the source, tokens,
    # first token in the round); empty sources own no tile, a source's last
    # tile is partial, and rounds above 32 tiles, one-kernel rounds and
    # cached rounds carry no records
    x = Ctx(lib, cfg(N=3, F=2, E=8, K=2, cap=4096))
    assert x.dispatch(0, 65) == 0 and x.dispatch(1, 0) == 0 and x.dispatch(2, 500) == 0
    assert x.receive(0)[0] == 0
    assert tiles(lib) == [(0, 0, 64, 0), (0, 64, 1, 64)] + [(2, 64 * i, 64, 65 + 64 * i) for i in range(7)] + \
        [(2, 448, 52, 513)]
    x.destroy()
    y = Ctx(lib, cfg(N=3, F=2, E=8, K=2, cap=4096))
    assert y.dispatch(0, 1) == 0 and y.dispatch(1, 2100) == 0 and y.dispatch(2, 1) == 0
    assert y.receive(0)[0] == 0
    t = tiles(lib)
    assert len(t) == 19 and t[0] == (0, 0, 1, 0) and t[-1] == (2, 0, 1, 2101)
    assert t[1:18] == [(1, 128 * i, 128 if i < 16 else 2100 - 2048, 1 + 128 * i) for i in range(17)]
    y.destroy()
    z = Ctx(lib, cfg(N=2, F=2, E=8, K=2, cap=8192))
    assert z.dispatch(0, 5000) == 0 and z.dispatch(1, 4000) == 0
    assert z.receive(0)[0] == 0
    assert tiles(lib) == []                  # 36 tiles of 256
    z.destroy()
    w = Ctx(lib, cfg(N=2, F=2, E=8, K=2, cap=64))
    assert w.dispatch(0, 30) == 0 and w.dispatch(1, 20) == 0
    assert w.receive(0)[0] == 0
    assert tiles(lib) == []                  # one-kernel dispatch
    w.destroy()
    v = Ctx(lib, cfg(N=1, F=2, E=8, K=2, cap=1024))
    v.full_round(T=(600,))
    assert tiles(lib) == [(0, 64 * i, 64 if i < 9 else 24, 64 * i) for i in range(10)]
    assert v.dispatch_cached(0, 600) == 0 and v.receive(0)[0] == 0
    assert tiles(lib) == []                  # cached dispatch: no layout kernel
    v.destroy()


def test_hip_failure_leaves_state(lib):
    x = Ctx(lib, cfg())
    for s in range(2):
        assert x.dispatch(s, 2) == 0
    lib.afd_fake_set_fail(1)
    try:
        assert x.receive(0)[0] == nat.AFD_E_HIP
    finally:
        lib.afd_fake_set_fail(0)
    st, r0, _ = x.receive(0)
    assert st == 0
    st, r1, _ = x.receive(1)
    assert x.reply(0, r0) == 0
    lib.afd_fake_set_fail(1)
    try:
        assert x.reply(1, r1) == nat.AFD_E_HIP                   # combine launch failed: reply not recorded
    finally:
        lib.afd_fake_set_fail(0)
    assert x.reply(1, r1) == 0
    x.destroy()


@pytest.mark.parametrize("mode", [1, 2])
def test_per_stage_round_launches(lib, mode):
    """Per-stage combine: each reply runs its partition's stage one, the
    round's last reply (whichever partition it is) its own stage one and
    stage two for every source in one launch; collects enqueue nothing."""
    c = cfg(N=2, F=3, E=6, K=2, H=512, cap=16, combine=mode)
    _, ws_once, _ = query(lib, cfg(N=2, F=3, E=6, K=2, H=512, cap=16), 16)
    x = Ctx(lib, c)
    prow = 512 * 2 if mode == 1 else 512 + 32
    assert x.ws - ws_once >= 3 * 2 * 16 * prow                  # partial rows in the workspace
    lib.afd_fake_log_clear()
    assert x.dispatch(0, 5) == 0 and x.dispatch(1, 4, out=0x7100000) == 0
    recs = [x.receive(f)[1] for f in range(3)]
    assert log(lib) == ["dispatch fused=1 ntok=9 nblk=1 T=5,4"]
    assert x.reply(2, recs[2]) == 0
    lg = log(lib)
    assert len(lg) == 1 and lg[0].startswith(f"partial f=2 ntok=9 prow={prow} base=")
    base = int(lg[0].split("base=")[1], 16)
    assert FAKE_WS < base < FAKE_WS + x.ws
    assert x.reply(0, recs[0]) == 0 and log(lib)[0].startswith("partial f=0")
    assert x.collect(0)[0] == nat.AFD_E_ORDER                    # partition 1 has not replied
    assert x.reply(1, recs[1]) == 0
    assert log(lib) == [f"last f=1 ntok=9 prow={prow} base={lg[0].split('base=')[1]} out=0x7000000,0x7100000"]
    st, res, stride = x.collect(1)
    assert st == 0 and res == 0x7100000 and stride == 512
    assert log(lib) == []
    assert x.collect(0)[0] == 0 and log(lib) == []
    # where source s's rows from partition f live
    ptr, rb = ctypes.c_void_p(), ctypes.c_int64()
    for (s_, f_) in [(0, 0), (1, 0), (0, 2), (1, 1)]:
        assert lib.afd_get_partials(x.ctx, s_, f_, ctypes.byref(ptr), ctypes.byref(rb)) == 0
        assert rb.value == prow and ptr.value == base + ((f_ * 2 + s_) * 16) * prow
    assert lib.afd_get_partials(x.ctx, 2, 0, ctypes.byref(ptr), None) == nat.AFD_E_ARG
    assert lib.afd_get_partials(x.ctx, 0, 3, ctypes.byref(ptr), None) == nat.AFD_E_ARG
    # stage two runs once, with the last reply's stage one
    assert x.dispatch(0, 0, out=0) == 0 and x.dispatch(1, 3) == 0
    recs = [x.receive(f)[1] for f in range(3)]
    log(lib)
    for f in (1, 2, 0):
        assert x.reply(f, recs[f]) == 0
    lg = log(lib)
    assert [m.split(" ")[:2] for m in lg] == [["partial", "f=1"], ["partial", "f=2"], ["last", "f=0"]]
    assert lg[2].endswith(" out=(nil),0x7000000")
    assert x.collect(0)[0] == 0 and x.collect(1)[0] == 0 and log(lib) == []
    # a round without tokens runs none
    assert x.dispatch(0, 0, out=0) == 0 and x.dispatch(1, 0, out=0) == 0
    recs = [x.receive(f)[1] for f in range(3)]
    for f in range(3):
        assert x.reply(f, recs[f]) == 0
    log(lib)
    assert x.collect(1)[0] == 0 and x.collect(0)[0] == 0 and log(lib) == []
    x.destroy()


def test_partials_refused_in_once_mode(lib):
    x = Ctx(lib, cfg())
    ptr = ctypes.c_void_p()
    assert lib.afd_get_partials(x.ctx, 0, 0, ctypes.byref(ptr), None) == nat.AFD_E_ARG
    x.destroy()


def test_per_stage_failed_launches_leave_state(lib):
    x = Ctx(lib, cfg(combine=1))
    for s in range(2):
        assert x.dispatch(s, 2) == 0
    recs = [x.receive(f)[1] for f in range(2)]
    lib.afd_fake_set_fail(1)
    try:
        assert x.reply(0, recs[0]) == nat.AFD_E_HIP               # stage one failed: reply not recorded
    finally:
        lib.afd_fake_set_fail(0)
    assert x.reply(0, recs[0]) == 0
    lib.afd_fake_set_fail(1)
    try:
        assert x.reply(1, recs[1]) == nat.AFD_E_HIP               # stage one + two failed: not recorded
    finally:
        lib.afd_fake_set_fail(0)
    assert x.collect(0)[0] == nat.AFD_E_ORDER
    assert x.reply(1, recs[1]) == 0
    assert x.collect(0)[0] == 0 and x.collect(1)[0] == 0
    x.destroy()


def test_cached_round(lib):
    """A cached dispatch reuses the last enqueued layout: its T per source and
    bucket, no ids, no host counts, and every source of the round alike."""
    x = Ctx(lib, cfg())
    assert x.dispatch_cached(0, 4) == nat.AFD_E_ORDER              # no layout yet
    x.full_round(T=(4, 3))
    lib.afd_fake_log_clear()
    assert x.dispatch_cached(0, 5) == nat.AFD_E_SHAPE              # T differs from the layout
    assert x.dispatch_cached(0, 4, bucket=8) == nat.AFD_E_ARG      # bucket differs
    assert x.dispatch_cached(0, 4, w=0) == nat.AFD_E_ARG           # weights required
    assert x.dispatch_cached(0, 4) == 0
    assert x.dispatch(1, 3) == nat.AFD_E_ORDER                     # mixed in one round
    assert x.dispatch_cached(1, 3) == 0
    assert log(lib) == []
    st, r0, _ = x.receive(0)
    assert st == 0 and log(lib) == ["dispatch cached ntok=7 T=4,3"]
    assert x.receive(1, rhc=1)[0] == nat.AFD_E_ARG                 # no host counts in a cached round
    st, r1, _ = x.receive(1)
    assert x.reply(0, r0) == 0 and x.reply(1, r1) == 0
    assert log(lib) == ["combine ntok=7 out=0x7000000,0x7000000"]
    assert x.collect(0)[0] == 0 and x.collect(1)[0] == 0
    # a new layout (different T) becomes the cached one
    x.full_round(T=(2, 6))
    assert x.dispatch_cached(0, 4) == nat.AFD_E_SHAPE
    assert x.dispatch_cached(0, 2) == 0 and x.dispatch_cached(1, 6) == 0
    lib.afd_fake_log_clear()
    assert x.receive(0)[0] == 0 and log(lib) == ["dispatch cached ntok=8 T=2,6"]
    x.destroy()


def test_cached_round_empty_and_fp8(lib):
    y = Ctx(lib, cfg(dtype=1))
    y.full_round(T=(0, 5))
    assert y.dispatch_cached(0, 0, out=0) == 0
    assert y.dispatch_cached(1, 5, scale=0) == nat.AFD_E_ARG       # FP8 needs scales
    assert y.dispatch_cached(1, 5, sst=1, ssg=5) == 0
    lib.afd_fake_log_clear()
    assert y.receive(0)[0] == 0 and log(lib) == ["dispatch cached ntok=5 T=0,5"]
    y.destroy()


def _info(lib, x):
    ri = nat.RoundInfo()
    assert lib.afd_get_round_info(x.ctx, ctypes.byref(ri)) == 0
    return ri


def test_round_info_names_the_dispatch_path(lib):
    """afd_get_round_info reports the kernels the executor runs: the
    one-kernel dispatch for small rounds, the tiled layout + scatter above its
    limits, the cached scatter, and the empty dispatch."""
    assert lib.afd_get_round_info(None, None) == nat.AFD_E_ARG
    c = cfg(E=8, K=2, cap=1024)
    x = Ctx(lib, c)
    ri = _info(lib, x)
    assert ri.round == 0 and ri.dispatch_path == 0
    x.full_round(T=(4, 3))
    ri = _info(lib, x)
    assert (ri.round, nat.DISPATCH_PATHS[ri.dispatch_path], ri.dispatch_kernels, ri.combine_kernels, ri.tokens) == \
        (1, "one_kernel", 1, 1, 7)
    x.full_round(T=(600, 3))                                  # more than 512 tokens: tiled
    ri = _info(lib, x)
    assert nat.DISPATCH_PATHS[ri.dispatch_path] == "tiled" and ri.dispatch_kernels == 2
    assert ri.tile_tokens == 64 and ri.layout_tiles == 11     # 640 + 64 slots in tiles of 64
    for s, T in enumerate((600, 3)):
        assert x.dispatch_cached(s, T) == 0
    recs = [x.receive(f)[1] for f in range(2)]
    ri = _info(lib, x)
    assert nat.DISPATCH_PATHS[ri.dispatch_path] == "cached" and ri.dispatch_kernels == 1 and ri.round == 3
    for f, rec in enumerate(recs):
        assert x.reply(f, rec) == 0
    for s in range(2):
        assert x.collect(s)[0] == 0
    x.full_round(T=(0, 0))
    ri = _info(lib, x)
    assert nat.DISPATCH_PATHS[ri.dispatch_path] == "empty" and ri.combine_kernels == 0
    x.destroy()
    y = Ctx(lib, cfg(E=8, K=2, cap=16, combine=2))
    y.full_round(T=(4, 0))
    ri = _info(lib, y)
    assert ri.combine_kernels == 2                            # a stage one, then stage one + stage two
    y.destroy()


def test_create_static(lib):
    """afd_create_static: the device's static scratch as the workspace, one
    context per device at a time, configs whose workspace exceeds the array
    refused, and every later call as on a context from afd_create."""
    c = cfg()
    ctx = ctypes.c_void_p()
    assert lib.afd_create_static(ctypes.byref(c), None) == nat.AFD_E_ARG
    big = cfg(N=16, F=1, E=8, K=2, H=16384, cap=2048)            # 1 GiB of single-partition inboxes
    assert lib.afd_create_static(ctypes.byref(big), ctypes.byref(ctx)) == nat.AFD_E_CAPACITY
    assert lib.afd_create_static(ctypes.byref(cfg(H=200)), ctypes.byref(ctx)) == nat.AFD_E_SHAPE
    lib.afd_fake_log_clear()
    assert lib.afd_create_static(ctypes.byref(c), ctypes.byref(ctx)) == 0
    assert log(lib)[0].startswith("init_static ws=0x100000000")
    other = ctypes.c_void_p()
    assert lib.afd_create_static(ctypes.byref(c), ctypes.byref(other)) == nat.AFD_E_ORDER
    x = Ctx.__new__(Ctx)
    x.lib, x.c, x.ctx = lib, c, ctx
    _, _, x.rb = query(lib, c, c.capacity)
    for f in range(2):
        assert lib.afd_bind_partition(ctx, f, 0x100000 * (f + 4), 0, 0x200000 + f * 0x1000, x.rb) == 0
    recs = x.full_round(T=(4, 3))
    assert recs[0].ends == (1 << 32) + 256                      # ends[] right after the error word's 256 bytes
    x.full_round(T=(2, 0))
    assert lib.afd_destroy(ctx) == 0
    assert lib.afd_create_static(ctypes.byref(c), ctypes.byref(other)) == 0   # free again
    assert lib.afd_destroy(other) == 0


def test_one_launch_dispatch_plan(lib):
    """AFD_DISPATCH_ONE_LAUNCH runs tiled rounds of at most 32 tiles and 256
    experts as one launch; small rounds keep the one-kernel dispatch, larger
    ones (more tiles, more experts) and cached rounds the other paths."""
    assert lib.afd_query(ctypes.byref(cfg(dispatch=3)), 8, None, None) == nat.AFD_E_SHAPE
    x = Ctx(lib, cfg(E=8, K=2, cap=8192, dispatch=nat.AFD_DISPATCH_ONE_LAUNCH))
    assert lib.afd_set_dispatch_wait(None, 5) == nat.AFD_E_ARG
    assert lib.afd_set_dispatch_wait(x.ctx, 77) == 0
    lib.afd_fake_log_clear()
    x.full_round(T=(4, 3))
    assert log(lib)[0].startswith("dispatch fused=1")
    x.full_round(T=(600, 3))
    assert log(lib)[0] == "dispatch onepass ntok=603 nblk=11 T=600,3 tile=64 wait=77"
    assert nat.DISPATCH_PATHS[_info(lib, x).dispatch_path] == "one_launch"
    x.full_round(T=(8192, 0))                                   # 32 tiles of 256: still one launch
    assert log(lib)[0].startswith("dispatch onepass ntok=8192 nblk=32")
    x.full_round(T=(8192, 1))                                   # 33 tiles: the split path
    assert log(lib)[0].startswith("dispatch fused=0 ntok=8193 nblk=33")
    for s, T in enumerate((8192, 1)):
        assert x.dispatch_cached(s, T) == 0
    recs = [x.receive(f)[1] for f in range(2)]
    assert log(lib)[0].startswith("dispatch cached")
    for f, rec in enumerate(recs):
        assert x.reply(f, rec) == 0
    for s in range(2):
        assert x.collect(s)[0] == 0
    x.destroy()
    y = Ctx(lib, cfg(E=512, F=2, K=2, cap=1024, dispatch=nat.AFD_DISPATCH_ONE_LAUNCH))
    lib.afd_fake_log_clear()
    y.full_round(T=(600, 3))                                    # more than 256 experts: the split path
    assert log(lib)[0].startswith("dispatch fused=0")
    y.destroy()


def test_timeout_reported_by_get_error(lib):
    x = Ctx(lib, cfg())
    code, s, t, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    lib.afd_fake_set_stall(1)
    args = (ctypes.byref(code), ctypes.byref(s), ctypes.byref(t), ctypes.byref(k))
    assert lib.afd_get_error(x.ctx, None, 0, *args) == nat.AFD_E_TIMEOUT
    assert lib.afd_get_error(x.ctx, None, 1, *args) == nat.AFD_E_TIMEOUT     # reported, then cleared
    assert lib.afd_get_error(x.ctx, None, 0, *args) == nat.AFD_OK
    assert lib.afd_status_string(nat.AFD_E_TIMEOUT)
    x.destroy()
