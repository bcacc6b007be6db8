"""GPU parity of the one-kernel dispatch's three forms of reading the ids:
two sources with eight 16-byte aligned ids per token (every thread holds
its tokens' ids in registers, up to two tokens per thread), at most two
sources otherwise, and any number of sources (ids copied into LDS).  The
contract allows ids at any 4-byte alignment, so the same rounds also run
with each source's ids moved 4 bytes off a 16-byte boundary.  Bar: layout,
rows, scales, weights bit-exact and the combine within tolerance (and, as
everywhere, expected bit-exact) against the oracle."""
import numpy as np
import pytest

import oracle
from synthetic import gen
from tests.test_gpu_parity import check_round

pytestmark = pytest.mark.gpu


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import harness
    return harness


# (seed, T per source, E, F, alpha, H, dtype, p_skip): eight ids per token,
# ragged and empty sources, rounds above 256 tokens (two per thread) up to
# the one-kernel limit of 512, power-of-two and other alignments
K8 = [
    (0, [128, 128], 128, 2, 64, 2048, "bf16", 0.0),
    (1, [300, 212], 128, 2, 64, 512, "bf16", 0.1),
    (2, [511, 1], 64, 4, 3, 256, "bf16", 0.2),
    (3, [0, 257], 16, 2, 1, 256, "bf16", 0.0),
    (4, [257, 0], 256, 1, 8, 1024, "fp8", 0.1),
    (5, [1, 1], 8, 2, 2, 256, "bf16", 0.0),
    (6, [200, 56], 32, 4, 5, 768, "fp8", 0.3),
    (7, [5], 96, 3, 128, 4096, "bf16", 0.0),
    (8, [256, 256], 248, 2, 16, 256, "bf16", 0.0),
    (9, [90, 333], 200, 5, 7, 512, "fp8", 0.05),
    (10, [64, 65], 128, 2, 64, 2048, "fp8", 0.0),
    (11, [420], 8, 1, 1, 256, "bf16", 0.5),
]


def _instance(case):
    seed, T, E, F, alpha, H, dtype, p_skip = case
    return gen.random_small(2100 + seed, N=len(T), F=F, E=E, K=8, alpha=alpha, T=T, H=H, p_skip=p_skip,
                            dtype=dtype, bucket=max(max(T), 1))


@pytest.mark.parametrize("case", K8, ids=lambda c: f"k8-{c[0]}-T{'_'.join(map(str, c[1]))}")
def test_eight_ids_per_token(case):
    h = _gpu()
    inst = _instance(case)
    print(f"[fused ids] {case}", flush=True)
    buf = h.make_buffer(inst)
    g = h.run_round(inst, buf)
    assert buf.round_info()["dispatch_path"] == "one_kernel"
    assert check_round(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0


def _moved(t, words):
    """A copy of the contiguous tensor t that starts `words` 4-byte words past
    a 16-byte boundary (same shape and contents)."""
    import torch
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    v = flat[words:words + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 4 * words % 16
    return v


# (workload or K8 case, sources whose ids move): the one-kernel dispatch with
# eight ids (the register form gives way to the LDS copy) and with two, the
# tiled layout kernel
MOVED = [("2a2f_decode", (0,)), ("2a2f_decode", (1,)), ("2a2f_decode", (0, 1)), ("tiny", (0,)),
         (1, (0, 1)), (2, (1,)), ("2a2f_skew_h4096", (0, 1)), ("1a3f_e96", (0,))]


@pytest.mark.parametrize("case", MOVED, ids=lambda c: f"{c[0]}-s{''.join(map(str, c[1]))}")
def test_ids_off_16_byte_boundary(case):
    h = _gpu()
    which, moved = case
    inst = gen.instance_by_name(which) if isinstance(which, str) else _instance(K8[which])
    print(f"[fused ids moved] {which} sources {moved}", flush=True)
    dev = h.upload(inst)
    dev = [(x, _moved(ids, 1) if s in moved else ids, w, sc) for s, (x, ids, w, sc) in enumerate(dev)]
    g = h.run_round(inst, dev=dev)
    assert check_round(inst, g, oracle.run_round(inst, rows_cap=g.receive_rows)) == 0
