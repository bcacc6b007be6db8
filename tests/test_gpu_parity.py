"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, on the
same seeded inputs.

Bar: ends, host counts, rows, FP8 scales, row weights and (harness) replies
bit-exact; combine within 1e-3 absolute + 1e-2 relative per element.  The
kernels accumulate in float32 in ascending k with separate multiply and add,
as the oracle does, so the combine is also expected to match bit for bit;
that stronger check is reported separately."""
import numpy as np
import pytest

import oracle
from synthetic import gen

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-3, 1e-2


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness
    return harness


def _concat(inst, attr):
    arrs = [getattr(s, attr) for s in inst.sources]
    return np.concatenate(arrs)


def live_ranges(ends, f, E_loc, alpha):
    prev = 0
    out = []
    for j in range(E_loc):
        st = (prev + alpha - 1) // alpha * alpha
        out.append((st, int(ends[f * E_loc + j])))
        prev = int(ends[f * E_loc + j])
    return out


def check_round(inst, g, ref, *, check_rows=True):
    cfg = inst.cfg
    E_loc = cfg.E // cfg.F
    lay = ref.layout
    for f in range(cfg.F):
        assert np.array_equal(g.ends[f], lay.ends[f * E_loc:(f + 1) * E_loc]), f"ends of partition {f}"
        if g.host_counts[f] is not None:
            assert list(g.host_counts[f]) == list(lay.host_counts[f * E_loc:(f + 1) * E_loc])
            assert g.receive_rows[f] == lay.rows_exact[f]
        if not check_rows:
            continue
        for st, en in live_ranges(lay.ends, f, E_loc, cfg.alpha):
            if en <= st:
                continue
            assert np.array_equal(g.rows[f][st:en], ref.rows[f][st:en]), f"rows p{f} [{st},{en})"
            assert np.array_equal(g.row_weights[f][st:en], ref.row_weights[f][st:en]), f"weights p{f}"
            if cfg.dtype == "fp8":
                assert np.array_equal(g.scales[f][st:en], ref.scales[f][st:en]), f"scales p{f}"
            assert np.array_equal(g.replies[f][st:en], ref.replies[f][st:en]), f"replies p{f}"
    out_ref = ref.out
    off = 0
    mism = 0
    for s, T in enumerate(cfg.T):
        got = gen.bf16_bits_to_f32(g.out[s].reshape(T, cfg.H)).astype(np.float64)
        want = gen.bf16_bits_to_f32(out_ref[off:off + T]).astype(np.float64)
        assert np.all(np.isfinite(got)), f"non-finite output of source {s}"
        bad = np.abs(got - want) > ATOL + RTOL * np.abs(want)
        assert not bad.any(), f"source {s}: {int(bad.sum())} elements out of tolerance"
        mism += int((g.out[s].reshape(T, cfg.H) != out_ref[off:off + T]).sum())
        off += T
    return mism


def _oracle_ref(inst, rows_cap):
    return oracle.run_round(inst, rows_cap=rows_cap)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_parity_workloads(name):
    h = _gpu()
    inst = gen.instance_by_name(name)
    print(f"[parity] {name}", flush=True)
    g = h.run_round(inst)
    ref = _oracle_ref(inst, g.receive_rows)
    mism = check_round(inst, g, ref)
    assert mism == 0, f"{mism} combine elements differ in the last bit from the oracle"


@pytest.mark.parametrize("name", ["tiny", "2a2f_decode", "1a3f_e96", "2a2f_fp8_prefill"])
def test_parity_read_host_counts(name):
    h = _gpu()
    inst = gen.instance_by_name(name)
    print(f"[parity rhc] {name}", flush=True)
    g = h.run_round(inst, rhc=True)
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0


SWEEP = [(i,) for i in range(24)]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"r{c[0]}")
def test_parity_random_small(case):
    h = _gpu()
    i = case[0]
    dtype = "fp8" if i % 4 == 3 else "bf16"
    H = [256, 512, 768, 1024][i % 4]
    inst = gen.random_small(i, H=H, dtype=dtype)
    print(f"[parity small] r{i} T={inst.cfg.T} E={inst.cfg.E} F={inst.cfg.F} K={inst.cfg.K} a={inst.cfg.alpha}",
          flush=True)
    g = h.run_round(inst, rhc=(i % 2 == 0))
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0


SPLIT = [(i,) for i in range(12)]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"m{c[0]}")
def test_parity_random_split_path(case):
    """Rounds above the one-kernel limits (more than 512 tokens, more than
    4096 ids or more than 256 experts) take the tiled layout + scatter path."""
    h = _gpu()
    i = case[0]
    rng = np.random.default_rng(77 + i)
    F = int(rng.choice([1, 2, 3, 4]))
    E = F * int(rng.choice([2, 8, 32, 128])) if i % 4 != 3 else 512
    E = min(E, 512) // F * F
    K = int(rng.choice([1, 4, 8, 12, 32])) if E >= 32 else int(rng.integers(1, min(8, E) + 1))
    K = min(K, E)
    N = int(rng.integers(1, 4))
    T = [int(rng.integers(0, 700)) for _ in range(N)]
    if sum(T) <= 512 and sum(T) * K <= 4096 and E <= 256:
        T[0] += 600
    bucket = max(T)
    alpha = int(rng.choice([1, 3, 16, 128]))
    dtype = "fp8" if i % 3 == 2 else "bf16"
    inst = gen.random_small(200 + i, N=N, F=F, E=E, K=K, alpha=alpha, T=T, H=256 if i % 2 else 512,
                            p_skip=0.1, dtype=dtype, bucket=bucket)
    print(f"[parity split] m{i} T={T} E={E} F={F} K={K} a={alpha} {dtype}", flush=True)
    g = h.run_round(inst, rhc=(i % 2 == 1))
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0


TILED = [(0, [5000, 4000], 256, 4, "bf16"), (1, [600], 8192, 8, "bf16"), (2, [9000], 256, 2, "fp8"),
         (3, [3000, 3000], 4096, 3, "bf16")]


@pytest.mark.parametrize("case", TILED, ids=lambda c: f"t{c[0]}")
def test_parity_tiled_path(case):
    """Larger tiled rounds: many tiles (more than 8192 tokens, so a tile's
    expert counts span more than 32 tiles), rows over 8 KB (the scatter loops
    over row chunks) and 8 KB rows with three ids per token."""
    h = _gpu()
    i, T, H, K, dtype = case
    inst = gen.random_small(400 + i, N=len(T), F=2, E=16, K=K, alpha=8, T=T, H=H, p_skip=0.1, dtype=dtype,
                            bucket=max(T))
    print(f"[parity tiled] t{i} T={T} H={H} K={K} {dtype}", flush=True)
    g = h.run_round(inst, rhc=(i % 2 == 0))
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0


@pytest.mark.parametrize("K", [12, 32])
def test_parity_fused_wide_topk(K):
    h = _gpu()
    inst = gen.random_small(300 + K, N=2, F=2, E=64, K=K, alpha=8, T=[40, 63], H=512, p_skip=0.1)
    print(f"[parity fused K={K}]", flush=True)
    g = h.run_round(inst)
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0


# (seed, tokens per source, H): the combine finds a token's output row from
# preloaded bases for sources 0 and 1 and from the offsets for later ones,
# and streams its stores when the output is at most 4 MiB.  Empty first or
# second sources, every token in a later source, and outputs at and just
# past the 4 MiB line.
SOURCES = [(0, [0, 300], 512), (1, [300, 0], 512), (2, [0, 1100], 2048), (3, [0, 0, 200], 512),
           (4, [100, 0, 0], 512), (5, [0, 0, 700, 5], 256), (6, [1024, 1024], 1024), (7, [1025, 1024], 1024),
           (8, [70, 0, 90], 768)]


@pytest.mark.parametrize("case", SOURCES, ids=lambda c: f"s{c[0]}")
def test_parity_combine_output_rows_of_every_source(case):
    h = _gpu()
    i, T, H = case
    inst = gen.random_small(900 + i, N=len(T), F=2, E=32, K=8, alpha=8, T=T, H=H, p_skip=0.1,
                            bucket=max(T))
    print(f"[parity sources] s{i} T={T} H={H} out={sum(T) * H * 2} B", flush=True)
    g = h.run_round(inst)
    ref = _oracle_ref(inst, g.receive_rows)
    assert check_round(inst, g, ref) == 0
