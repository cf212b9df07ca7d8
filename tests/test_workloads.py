"""Tests of the seeded input generators (CPU only): determinism, layouts, NaN
tails, block permutation, FP8 scales, bf16 rounding, and the ragged length
law against the horizon-average load B(mu_P + mu_D) of "Theoretically Optimal
Attention/FFN Ratios in Disaggregated LLM Serving" (probabilistic workload
model, horizon-average token load)."""

import numpy as np
import torch

from workloads import bf16_round_bits, config_case, make_decode_case, ragged_lengths


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.5e-39, 3.4e38], np.float32)])
    ours = bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_same_seed_same_case():
    a = make_decode_case(3, batch=2, ctx_lens=[100, 5], hq=64, hkv=1, d=256)
    b = make_decode_case(3, batch=2, ctx_lens=[100, 5], hq=64, hkv=1, d=256)
    for f in ("q", "k_cache", "v_cache", "block_table", "ctx_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_paged_layout_table_and_tails():
    c = make_decode_case(4, batch=3, ctx_lens=[130, 0, 64], hq=64, hkv=2, d=192)
    assert c.k_cache.shape == (3 + 0 + 1, 2, 64, 192)
    assert c.v_cache.shape == (4, 2, 192, 64)
    assert c.block_table.shape == (3, 3)
    assert sorted(c.block_table[c.block_table >= 0].tolist()) == [0, 1, 2, 3]
    assert np.all(c.block_table[1] == -1) and c.block_table[2, 1] == -1
    last = c.block_table[0, 2]
    assert np.all(c.k_cache[last, :, 2:, :] == 0x7FC0)
    assert np.all(c.v_cache[last, :, :, 2:] == 0x7FC0)
    assert not np.any(c.k_cache[last, :, :2, :] == 0x7FC0)


def test_fp8_scales_are_absmax_over_448_and_codes_saturate():
    c = make_decode_case(5, batch=2, ctx_lens=[64, 100], hq=64, hkv=1, d=256, kv_format="e4m3")
    assert c.k_cache.dtype == np.uint8
    valid = c.k_cache[c.block_table[c.block_table >= 0]]
    codes = valid[(valid & 0x7F) != 0x7F]
    # the largest magnitude code is 448 (0x7E) exactly once per head at least
    assert (codes & 0x7F).max() == 0x7E
    assert c.k_scale.shape == (1,) and c.k_scale[0] > 0


def test_contiguous_layout():
    c = config_case(1)
    assert c.block_table is None
    assert c.k_cache.shape == (2, 128, 1, 256) and c.v_cache.shape == (2, 1, 256, 128)
    assert c.k_cache.dtype == np.float32
    assert np.all(np.isnan(c.k_cache[1, 77:])) and np.all(np.isnan(c.v_cache[1, :, :, 77:]))
    assert not np.any(np.isnan(c.k_cache[1, :77]))


def test_ragged_length_law_matches_horizon_average():
    # mu_P = (1024 + 8192) / 2, mu_D = (1 - p) / p with p = 1/1024
    draw = ragged_lengths(128)
    means = [draw(np.random.default_rng(s)).mean() for s in range(200)]
    expect = 4608 + 1023
    se = np.std(means) / np.sqrt(len(means))
    assert abs(np.mean(means) - expect) < 4 * se + 5
    lens = draw(np.random.default_rng(3))
    assert lens.min() >= 1024 and lens.max() <= 32768
