"""GPU parity of the per-group (GQA) decode kernel over an FP8 E4M3 cache
against the fp64 oracle: 16 query heads per KV group, width 192 (the Step-5
layer, "Step-5-Preview: Sparse GQA, Indexer und KV-Speicher") or 256, one
fp32 scale per KV group (stored value = code x scale), codes widened to bf16
MFMA operands in the kernel.

Covers ragged lengths straddling the window and the 64-key blocks with NaN
codes past each length, windows 0 / 512 / 100, split counts, fp32 output, the
contiguous cache, block permutations bit for bit, and an exact check of every
finite code: with a one-hot attention pattern the output row is exactly the
decoded V row."""

import numpy as np
import pytest
import torch

from oracle import decode_attention
from workloads import make_decode_case

from gpu_helpers import assert_parity, run_decode, to_device

pytestmark = pytest.mark.gpu

LENS = [1, 63, 511, 512, 513, 700, 2000, 0]


def oracle(case):
    return decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                            **case.oracle_kwargs())


@pytest.mark.parametrize("window", [0, 512, 100])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_step5_shape_fp8(window, splits):
    print(f"gqa fp8 d=192 window={window} splits={splits}", flush=True)
    case = make_decode_case(150 + window, batch=len(LENS), ctx_lens=LENS, hq=64, hkv=4, d=192,
                            kv_format="e4m3", window=window)
    got = run_decode(case, to_device(case), num_splits=splits)
    assert_parity(got, oracle(case), "e4m3", f"gqa fp8 d=192 window={window} splits={splits}")


@pytest.mark.parametrize("window", [0, 77])
def test_width256_fp8(window):
    case = make_decode_case(160 + window, batch=4, ctx_lens=[65, 1000, 0, 257], hq=32, hkv=2,
                            d=256, kv_format="e4m3", window=window, scale=1 / 16)
    got = run_decode(case, to_device(case), num_splits=2)
    assert_parity(got, oracle(case), "e4m3", f"gqa fp8 d=256 window={window}")


def test_contiguous_cache_and_fp32_output_fp8():
    case = make_decode_case(170, batch=5, ctx_lens=[1, 130, 640, 0, 1999], hq=64, hkv=4, d=192,
                            kv_format="e4m3", out_format="f32", paged=False, window=512)
    got = run_decode(case, to_device(case), num_splits=0)
    assert got.dtype == torch.float32
    assert_parity(got, oracle(case), "e4m3", "gqa fp8 contiguous, fp32 out")


@pytest.mark.parametrize("splits", [1, 3])
def test_fp8_gqa_block_permutation_is_bit_exact(splits):
    kw = dict(batch=4, ctx_lens=[777, 64, 2049, 513], hq=64, hkv=4, d=192, kv_format="e4m3")
    a = make_decode_case(171, shuffle=False, **kw)
    b = make_decode_case(171, shuffle=True, **kw)
    assert not np.array_equal(a.block_table, b.block_table)
    ga = run_decode(a, to_device(a), num_splits=splits).clone()
    gb = run_decode(b, to_device(b), num_splits=splits).clone()
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


@pytest.mark.parametrize("d,hq,hkv", [(192, 64, 4), (256, 32, 2)])
def test_every_finite_code_decodes_exactly(d, hq, hkv):
    """q = 1, K code 448 on key j* and 0 on every other key: the logit gap
    (d x 448 x scale, over 6000) underflows every other weight to exactly 0,
    so with unit scales each output row is the decoded V row at j*.  Across
    the groups, V channel c of group g holds code (c + 64 g) mod 256, which
    covers every finite code."""
    L, jstar = 1500, 777
    case = make_decode_case(172, batch=1, ctx_lens=[L], hq=hq, hkv=hkv, d=d, kv_format="e4m3")
    case.q[:] = 0x3F80                                   # bf16 1.0
    case.k_scale[:] = 1.0
    case.v_scale[:] = 1.0
    blk, row = case.block_table[0, jstar // 64], jstar % 64
    for i in range((L + 63) // 64):
        b = case.block_table[0, i]
        rows = np.arange(64)[np.arange(64) < L - 64 * i]
        case.k_cache[b, :, rows, :] = 0
    case.k_cache[blk, :, row, :] = 0x7E                  # 448
    for g in range(hkv):
        codes = ((np.arange(d) + 64 * g) % 256).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0                # NaN codes -> 0
        case.v_cache[blk, g, :, row] = codes
    got = run_decode(case, to_device(case), num_splits=1).float().cpu().numpy()
    np.testing.assert_array_equal(got, oracle(case).astype(np.float32))
