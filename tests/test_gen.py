"""Pins for the seeded input generator (CPU only).

The generator's number formats are checked against torch's CPU casts (a
library routine); its routing draws against the properties the workloads
state (distinct ids per token, the -1 rate, Zipf popularity)."""
import numpy as np
import pytest
import torch

from synthetic import gen


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties: bit patterns whose low half is 0x8000 with both parities
    ties = (np.arange(2000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)
    v = np.concatenate([v, ties, np.array([0.0, -0.0, 1e-40, -1e-40, 3.3e38], np.float32)])
    ours = gen.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gen.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = gen.e4m3_bits_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_including_ties():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(100000) * 100).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    # every midpoint between adjacent finite codes (exact ties), both signs
    pos = gen.e4m3_bits_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, pos.astype(np.float32), np.array([448.00003, 460.0], np.float32)])
    ours = gen.f32_to_e4m3_bits(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_block_quantisation_round_trip_bound():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 512), dtype=np.float32)
    q, scale = gen.quantize_fp8_blocks(x)
    assert q.dtype == np.uint8 and scale.shape == (16, 4)
    xr = gen.e4m3_bits_to_f32(q).reshape(16, 4, 128) * scale[:, :, None]
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 in the normal range
    amax = np.abs(x.reshape(16, 4, 128)).max(axis=2, keepdims=True)
    err = np.abs(xr - x.reshape(16, 4, 128))
    assert np.all(err <= amax * 2.0 ** -4 + 1e-12)
    assert np.all(np.abs(gen.e4m3_bits_to_f32(q)) <= 448.0)


@pytest.mark.parametrize("name", gen.WORKLOADS)
def test_workload_shapes_and_routes(name):
    inst = gen.instance_by_name(name)
    cfg = inst.cfg
    for src, T in zip(inst.sources, cfg.T):
        assert src.ids.shape == (T, cfg.K) and src.ids.dtype == np.int32
        assert src.weights.shape == (T, cfg.K) and src.weights.dtype == np.float32
        live = src.ids[src.ids >= 0]
        assert live.size == 0 or (live.min() >= 0 and live.max() < cfg.E)
        for row in src.ids:
            r = row[row >= 0]
            assert len(set(r.tolist())) == len(r)          # distinct per token
        np.testing.assert_allclose(src.weights.sum(axis=1), 1.0, rtol=1e-5)
        if cfg.dtype == "fp8":
            assert src.x.dtype == np.uint8 and src.scale.shape == (T, cfg.H // 128)
        else:
            assert src.x.dtype == np.uint16 and src.x.shape == (T, cfg.H)


def test_skip_rate_and_determinism():
    a, b = gen.cfg_ratio_pair()
    rng = np.random.default_rng(4)
    ia = gen.generate(a, rng)
    ib = gen.generate(b, rng)
    rate = np.mean(np.concatenate([s.ids.ravel() for s in ib.sources]) == -1)
    assert abs(rate - 0.05) < 0.01
    assert gen.instance_by_name("3a1f_e96_view").digests() == ib.digests()
    assert gen.instance_by_name("1a3f_e96").digests() == ia.digests()


def test_zipf_popularity():
    inst = gen.instance_by_name("2a2f_skew_h4096")
    ids = np.concatenate([s.ids for s in inst.sources])
    counts = np.bincount(ids.ravel(), minlength=128)
    # the most popular expert is chosen by most tokens (Zipf(1) over 128 with
    # 8 draws without replacement), far above the uniform mean of 64 per expert
    assert counts.max() > 0.7 * ids.shape[0]
    assert counts.max() > 8 * counts.mean()
