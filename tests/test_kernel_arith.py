"""CPU checks of arithmetic shortcuts the kernels take, in float32 as the
device computes it.

The one-kernel dispatch finds an expert's partition as
int((e + 0.5) * rcp(E_loc)) instead of an integer division.  The hardware
reciprocal is accurate to 1 ulp, so the check runs every E_loc of the
one-kernel path (1..256) and every e below 2^16 with the correctly rounded
reciprocal and its neighbours up to 2 ulp away."""
import numpy as np


def test_partition_without_division():
    e = np.arange(1 << 16, dtype=np.int64)
    x = (e.astype(np.float32) + np.float32(0.5)).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), e + 0.5)        # exact in float32
    for E_loc in range(1, 257):
        want = e // E_loc
        r = np.float32(1.0) / np.float32(E_loc)
        for ulps in (-2, -1, 0, 1, 2):
            rr = r
            step = np.float32(np.inf) if ulps > 0 else np.float32(-np.inf)
            for _ in range(abs(ulps)):
                rr = np.nextafter(rr, step, dtype=np.float32)
            got = (x * rr).astype(np.float32).astype(np.int64)    # product rounded to float32, truncated
            assert np.array_equal(got, want), (E_loc, ulps)
