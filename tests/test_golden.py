"""Values the afdEP-comm design page prints, as fixtures under tests/golden/:

  * byte_model_3a1f.txt: the byte volumes of its 3:1 analysis, against the
    byte model of bench.py;
  * fp8_reply_row_bytes.txt: the FP8 reply row size of section 19 (4,128 B
    at H = 4096, and the size reductions at 4096, 7168 and 8192), against the
    oracle's FP8 partial row and the library's partial row size."""
import ctypes
import os

import bench
import oracle
from synthetic import gen

HERE = os.path.dirname(os.path.abspath(__file__))


def _fixture():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "byte_model_3a1f.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = int(v)
    return vals


def test_byte_model_matches_design_page_3a1f():
    f = _fixture()
    cfg = gen.Config("3a1f_page", 0, [f["tokens_per_source"]] * f["sources"], f["hidden"], 128, 1, f["topk"], 1)
    L = sum(cfg.T) * cfg.K                      # every choice is live on the single FFN
    t = bench.byte_terms(cfg, L)
    assert round(t["rows_write"] / 1e6) == f["expanded_rows_mb"]
    assert round(t["replies_read"] / 1e6) == f["expanded_rows_mb"]
    assert round(t["x_read"] / 1e6) == f["dispatch_payload_mb"]
    total = bench.round_bytes(cfg, L)["total"]
    assert total == sum(t.values())


def _fp8_rows():
    rows = []
    for line in open(os.path.join(HERE, "golden", "fp8_reply_row_bytes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            H, fp8, bf16, pct = line.split()
            rows.append((int(H), None if fp8 == "-" else int(fp8), None if bf16 == "-" else int(bf16), float(pct)))
    return rows


def test_fp8_reply_row_bytes_match_design_page():
    rows = _fp8_rows()
    assert [r[0] for r in rows] == [4096, 7168, 8192]
    for H, fp8, bf16, pct in rows:
        got = oracle.fp8_row_bytes(H)
        if fp8 is not None:
            assert got == fp8
            assert bf16 == 2 * H + 64
        assert round(100.0 * (1.0 - got / (2 * H + 64)), 1) == pct, H


def test_library_partial_row_bytes_match_design_page():
    """The library's FP8 partial rows (per-stage FP8 combine) have the page's
    size; checked through the host core over the recording backend."""
    from combine_layout_amd import _native as nat
    lib = nat.load_fake()
    for H, fp8, _, _ in _fp8_rows():
        cfg = nat.Config(2, 2, 16, 4, H, 1, 8, nat.AFD_BF16, nat.AFD_COMBINE_PER_STAGE_FP8)
        ws = ctypes.c_size_t(0)
        assert lib.afd_query(ctypes.byref(cfg), 8, ctypes.byref(ws), None) == 0
        ctx = ctypes.c_void_p(0)
        # the recording backend never touches the workspace: a fake, aligned address
        assert lib.afd_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), ws.value, ctypes.byref(ctx)) == 0
        ptr, rb = ctypes.c_void_p(0), ctypes.c_int64(0)
        assert lib.afd_get_partials(ctx, 0, 1, ctypes.byref(ptr), ctypes.byref(rb)) == 0
        assert rb.value == oracle.fp8_row_bytes(H)
        if fp8 is not None:
            assert rb.value == fp8
        lib.afd_destroy(ctx)
