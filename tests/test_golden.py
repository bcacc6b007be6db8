"""The byte model of bench.py against the byte volumes the afdEP-comm design
page prints for its 3:1 analysis (tests/golden/byte_model_3a1f.txt)."""
import os

import bench
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
