"""GPU parity with strided FP8 scale views (through the C ABI).

The API contract page ("Roles and tensors") takes FP32 block-128 scales
[T, H/128] and supports strided scale views.  Every dispatch kernel reads
scale (t, b) at t * stride_t + b * stride_g; these rounds pass views whose
strides differ from the dense (H/128, 1): a column-major view, a view whose
rows are padded (stride_t > H/128, the padding filled with NaN so a wrong
index shows), and a column-major view of a padded buffer.  The one-kernel
dispatch, the tiled layout + scatter and the cached scatter all run, each
compared bit for bit (scales, rows, ends) with the CPU oracle on the same
values."""
import dataclasses

import pytest

import oracle
from synthetic import gen

pytestmark = pytest.mark.gpu

VIEWS = ["column_major", "padded_rows", "column_major_padded"]


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness
    return harness


def _view(sc, kind):
    """A strided view holding the values of the dense [T, G] scales `sc`."""
    import torch
    T, G = sc.shape
    if kind == "column_major":
        v = sc.t().contiguous().t()                         # strides (1, T)
    elif kind == "padded_rows":
        buf = torch.full((T, G + 5), float("nan"), dtype=torch.float32, device=sc.device)
        buf[:, :G] = sc
        v = buf[:, :G]                                      # strides (G + 5, 1)
    else:
        buf = torch.full((G, T + 3), float("nan"), dtype=torch.float32, device=sc.device)
        buf[:, :T] = sc.t()
        v = buf.t()[:T]                                     # strides (1, T + 3)
    assert v.shape == (T, G) and v.stride() != (G, 1) and bool((v == sc).all())
    return v


def _dev_with_views(h, inst, kind):
    dev = h.upload(inst)
    return [(x, ids, w, _view(sc, kind) if sc.shape[0] else sc) for x, ids, w, sc in dev]


# (case, tokens per source, H): one-kernel dispatch (rounds of at most 512
# tokens), the tiled path with few and with many layout tiles, and rows with
# more scale blocks than a wavefront has lanes.
CASES = [("one_kernel", [40, 0, 63], 1024), ("tiled", [700, 300], 512), ("tiled_many", [5000, 4000], 256),
         ("tiled_wide", [600], 16384)]


@pytest.mark.parametrize("kind", VIEWS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_strided_scale_views(case, kind):
    h = _gpu()
    from tests.test_gpu_parity import check_round
    name, T, H = case
    inst = gen.random_small(1300 + len(name), N=len(T), F=2, E=32, K=8, alpha=16, T=T, H=H, p_skip=0.1,
                            dtype="fp8", bucket=max(T))
    print(f"[scale views] {name} {kind} T={T} H={H}", flush=True)
    g = h.run_round(inst, dev=_dev_with_views(h, inst, kind))
    assert check_round(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0


@pytest.mark.parametrize("kind", VIEWS)
@pytest.mark.parametrize("T", [[40, 63], [700, 300]], ids=["one_kernel_layout", "tiled_layout"])
def test_strided_scale_views_cached(T, kind):
    """The cached scatter reads the new round's scales through their strides."""
    h = _gpu()
    from tests.test_gpu_parity import check_round
    a = gen.random_small(1310, N=len(T), F=2, E=32, K=8, alpha=16, T=T, H=1024, p_skip=0.1, dtype="fp8",
                         bucket=max(T))
    b = gen.generate(dataclasses.replace(a.cfg, seed=a.cfg.seed + 1000))
    buf = h.make_buffer(a)
    print(f"[scale views cached] {kind} T={T}", flush=True)
    h.run_round(a, buf, keep_arrays=False)
    g = h.run_round(b, buf, dev=_dev_with_views(h, b, kind), cached=True)
    hyb = gen.Instance(b.cfg, [dataclasses.replace(y, ids=x.ids) for x, y in zip(a.sources, b.sources)])
    assert check_round(hyb, g, oracle.run_round(hyb, rows_cap=g.receive_rows)) == 0


def test_strided_scale_views_fp8_prefill():
    """The FP8 prefill workload (2 x 2048 tokens, H2048, E128 top-8) with
    column-major scales."""
    h = _gpu()
    from tests.test_gpu_parity import check_round
    inst = gen.instance_by_name("2a2f_fp8_prefill")
    print("[scale views] 2a2f_fp8_prefill column_major", flush=True)
    g = h.run_round(inst, dev=_dev_with_views(h, inst, "column_major"))
    assert check_round(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
