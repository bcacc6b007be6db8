"""Pins for the oracle's configuration and shape check (CPU only).

Step one of a round validates the configuration against the API contract
page ("Roles and tensors"): H a multiple of 256, K <= min(32, E), experts
split evenly over the FFN partitions, T <= bucket <= capacity, and (this
build's readings) alignment >= 1, at least one source and partition, and a
bucket of at least one token.  The pins are cases taken from those passages:
every workload shape the pages measure is accepted, each boundary value the
rules allow is accepted, and each rule broken alone is rejected."""
import dataclasses

import pytest

import oracle
from synthetic import gen

# A valid base: the decode workload's shape (2 sources, E128 over 2 FFN
# partitions, top-8, H2048, alignment 64, capacity bucket 2048).
BASE = dict(T=[128, 128], bucket=2048, capacity=2048, E=128, F=2, K=8, H=2048, alpha=64)


def _ok(**kw):
    a = dict(BASE)
    a.update(kw)
    return oracle.check_config(a["T"], a["bucket"], a["capacity"], a["E"], a["F"], a["K"], a["H"], a["alpha"])


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_page_workloads_accepted(name):
    c = gen.instance_by_name(name).cfg
    assert oracle.check_config(c.T, c.bucket, c.capacity, c.E, c.F, c.K, c.H, c.alpha)


# Boundary values each rule allows.
ACCEPT = [
    dict(H=256),                             # smallest multiple of 256
    dict(H=7168),                            # DeepSeek-V3's hidden size, 28 * 256
    dict(H=4096),
    dict(K=32, E=64, F=2),                   # K = 32 <= E
    dict(K=8, E=8, F=1),                     # K = E <= 32
    dict(K=1),
    dict(E=96, F=3),                         # the E96 layouts: 32 experts per partition
    dict(E=96, F=1),
    dict(E=128, F=128, K=8),                 # one expert per partition
    dict(alpha=1),
    dict(T=[2048, 2048]),                    # T = bucket = capacity
    dict(T=[0, 0]),                          # empty sources
    dict(T=[5], bucket=5, capacity=2048),    # bucket below capacity
    dict(T=[3, 0, 7], bucket=8, capacity=8),
]

# One rule broken, everything else valid.
REJECT = [
    dict(H=128),                             # not a multiple of 256
    dict(H=384),                             # a multiple of 128 but not of 256
    dict(H=2000),
    dict(H=0),
    dict(K=0),
    dict(K=33, E=64, F=2),                   # K > 32
    dict(K=9, E=8, F=1),                     # K > E
    dict(E=96, F=5),                         # experts do not split evenly
    dict(E=128, F=3),
    dict(E=0),
    dict(F=0),
    dict(alpha=0),
    dict(T=[129, 128], bucket=128, capacity=2048),   # T > bucket
    dict(bucket=4096, capacity=2048),                # bucket > capacity
    dict(T=[-1, 128]),
    dict(T=[0, 0], bucket=0, capacity=2048),
    dict(T=[]),
]


@pytest.mark.parametrize("kw", ACCEPT, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_boundary_values_accepted(kw):
    assert _ok(**kw)


@pytest.mark.parametrize("kw", REJECT, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_each_broken_rule_rejected(kw):
    assert not _ok(**kw)


def test_run_round_validates():
    """The whole-round oracle refuses an instance that breaks a rule."""
    inst = gen.instance_by_name("tiny")
    bad = gen.Instance(dataclasses.replace(inst.cfg, bucket=4, capacity=8), inst.sources)   # T = 8 > bucket
    with pytest.raises(ValueError):
        oracle.run_round(bad)
    oracle.run_round(inst)


def test_config_pins_all():
    """Every pin above in one call (the planted-mistake test runs this)."""
    for name in gen.WORKLOADS:
        test_page_workloads_accepted(name)
    for kw in ACCEPT:
        assert _ok(**kw), kw
    for kw in REJECT:
        assert not _ok(**kw), kw
