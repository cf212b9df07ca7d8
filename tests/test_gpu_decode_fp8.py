"""GPU parity of MFA decode attention over an FP8 E4M3 cache (per-KV-head fp32
scales, codes converted to bf16 on the way to LDS) against the fp64 oracle.

Covers ragged lengths with NaN tail codes, every split count, fp32 output, the
contiguous cache, the windowed path, the full-size 256 x 4096 batch on
sampled slots, and a bit-exact check of the conversion of every finite code:
with a one-hot attention pattern the output is exactly the decoded V row."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention
from workloads import make_decode_case
from workloads.device_gen import make_device_case

from gpu_helpers import assert_parity, run_decode, to_device

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 130, 1000, 0, 4096, 4033]


def oracle(case, slots=None):
    return decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                            slots=slots, **case.oracle_kwargs())


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_fp8_paged_ragged(splits):
    case = make_decode_case(90, batch=len(RAGGED), ctx_lens=RAGGED, hq=64, hkv=1, d=256,
                            kv_format="e4m3", scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits)
    assert_parity(got, oracle(case), "e4m3", f"fp8 splits={splits}")


def test_fp8_fp32_output_and_contiguous_cache():
    case = make_decode_case(91, batch=4, ctx_lens=[5, 640, 0, 1111], hq=64, hkv=1, d=256,
                            kv_format="e4m3", paged=False, scale=1 / 16)
    t = to_device(case, out_format="f32")
    got = run_decode(case, t)
    assert got.dtype == torch.float32
    assert_parity(got, oracle(case), "e4m3", "fp8 contiguous, fp32 out")


@pytest.mark.parametrize("window", [1, 300])
def test_fp8_window(window):
    case = make_decode_case(92, batch=5, ctx_lens=[1, 64, 299, 1500, 4000], hq=64, hkv=1,
                            d=256, kv_format="e4m3", window=window, scale=1 / 16)
    t = to_device(case)
    for splits in (0, 3):
        got = run_decode(case, t, num_splits=splits)
        assert_parity(got, oracle(case), "e4m3", f"fp8 window={window} splits={splits}")


@pytest.mark.parametrize("jstar,splits", [(0, 1), (77, 0), (1000, 3), (1999, 4)])
def test_every_finite_code_decodes_exactly(jstar, splits):
    """q = 1, K code 448 on key j* and 0 elsewhere: the logit gap of
    256 * 448 / 16 = 7168 underflows every other weight to exactly 0, so with
    unit scales the output row equals the decoded V row, which holds every
    finite code."""
    L = 2000
    case = make_decode_case(93, batch=1, ctx_lens=[L], hq=64, hkv=1, d=256,
                            kv_format="e4m3", scale=1 / 16)
    case.q[:] = 0x3F80                                   # bf16 1.0
    case.k_scale[:] = 1.0
    case.v_scale[:] = 1.0
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                    # NaN codes -> 0
    blk, row = case.block_table[0, jstar // 64], jstar % 64
    valid_rows = np.arange(64)
    for i in range((L + 63) // 64):
        b = case.block_table[0, i]
        rows = valid_rows[valid_rows < L - 64 * i]
        case.k_cache[b, 0, rows, :] = 0
    case.k_cache[blk, 0, row, :] = 0x7E                  # 448
    case.v_cache[blk, 0, :, row] = codes                 # channel c holds code c
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits).float().cpu().numpy()
    ref = oracle(case)
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def test_config4_full_size_sampled_slots():
    """256 slots x 4096 keys, E4M3 K/V with per-head scales (drawn on the device)."""
    dc = make_device_case(4, batch=256, ctx_lens=[4096] * 256, hq=64, hkv=1, d=256,
                          kv_format="e4m3", scale=1 / 16, name="c4")
    out = torch.full((256, 64, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_decode_attention(dc.q, dc.k, dc.v, dc.table, dc.lens, out, dc.scale,
                             k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    slots = [0, 100, 255]
    sub = dc.host_slots(slots)
    ref = decode_attention(sub.q, sub.k_cache, sub.v_cache, sub.ctx_lens, sub.scale,
                           **sub.oracle_kwargs())
    assert_parity(out[slots], ref, "e4m3", "config 4 sampled")
