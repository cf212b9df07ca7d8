"""GPU parity of the GQA / sliding-window entry (mfa_decode_attention_gqa)
against the fp64 oracle.

Shapes: the Step-5 GQA layer (64 query heads, 4 KV groups, width 192; local
layers attend to a 512-token window, the global layer to everything), a
16-head-per-group width-256 variant, and the MQA shape (64 heads, one KV
head, width 256) with a window, which runs the shared-tile kernel's windowed
path.  Ragged lengths straddle the window and the 64-key blocks; tail rows
past each length are NaN.  The full-size layer (32 slots x 32768 keys) is
drawn on the device and checked on every slot; block permutations must leave
the output bit for bit unchanged.
"""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention
from workloads import make_decode_case
from workloads.device_gen import make_device_case

from gpu_helpers import assert_parity, run_decode, to_device

pytestmark = pytest.mark.gpu

LENS = [1, 63, 511, 512, 513, 700, 2000, 0]


def oracle(case, slots=None, **over):
    kw = case.oracle_kwargs()
    kw.update(over)
    return decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                            slots=slots, **kw)


@pytest.mark.parametrize("window", [512, 0, 100])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_step5_gqa_shape(window, splits):
    case = make_decode_case(50 + window, batch=len(LENS), ctx_lens=LENS, hq=64, hkv=4, d=192,
                            window=window)
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits)
    assert_parity(got, oracle(case), "bf16", f"gqa d=192 window={window} splits={splits}")


@pytest.mark.parametrize("window", [0, 77])
def test_group16_width256(window):
    case = make_decode_case(60, batch=4, ctx_lens=[65, 1000, 0, 257], hq=32, hkv=2, d=256,
                            window=window, scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t, num_splits=2)
    assert_parity(got, oracle(case), "bf16", f"gqa d=256 window={window}")


@pytest.mark.parametrize("window", [1, 64, 300, 4096])
def test_mqa_shape_with_window(window):
    """64 heads on one KV head through the GQA entry: the shared-tile kernel's
    windowed path (the first page moves with the length)."""
    case = make_decode_case(70, batch=6, ctx_lens=[1, 64, 65, 300, 1500, 4000], hq=64, hkv=1,
                            d=256, window=window, scale=1 / 16)
    t = to_device(case)
    for splits in (0, 1, 4):
        got = run_decode(case, t, num_splits=splits)
        assert_parity(got, oracle(case), "bf16", f"mqa window={window} splits={splits}")


def test_window_covering_the_context_equals_dense_bit_exactly():
    case = make_decode_case(80, batch=3, ctx_lens=[100, 511, 512], hq=64, hkv=4, d=192,
                            window=0)
    t = to_device(case)
    dense = run_decode(case, t, num_splits=1).clone()
    wide = run_decode(case, t, num_splits=1, window=512)
    assert torch.equal(dense.view(torch.int16), wide.view(torch.int16))


def test_window_of_one_returns_the_last_value_row_exactly():
    case = make_decode_case(81, batch=3, ctx_lens=[1, 640, 1000], hq=64, hkv=4, d=192,
                            window=1)
    t = to_device(case)
    got = run_decode(case, t).float().cpu().numpy()
    ref = oracle(case)
    np.testing.assert_array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("window", [512, 0])
def test_step5_full_size_every_slot(window):
    """32 slots x 32768 keys, 4 KV groups of width 192 (1.6 GB of bf16 K/V),
    local (512-key window) and global (dense) layer; every slot against the
    oracle, copied back eight slots at a time."""
    dc = make_device_case(5, batch=32, ctx_lens=[32768] * 32, hq=64, hkv=4, d=192,
                          window=window, name="step5")
    out = torch.full((32, 64, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_decode_attention_gqa(dc.q, dc.k, dc.v, dc.table, dc.lens, out, dc.scale,
                                 window=window)
    torch.cuda.synchronize()
    refs = []
    for s0 in range(0, 32, 8):
        sub = dc.host_slots(list(range(s0, s0 + 8)))
        refs.append(decode_attention(sub.q, sub.k_cache, sub.v_cache, sub.ctx_lens, sub.scale,
                                     **sub.oracle_kwargs()))
        del sub
    assert_parity(out, np.concatenate(refs), "bf16", f"step5 full window={window}",
                  per_slot=True)
    del dc


@pytest.mark.parametrize("window", [0, 512])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_gqa_block_permutation_is_bit_exact(window, splits):
    # Step-5 shape (4 groups of width 192): the same logical cache in the
    # pool's identity order and shuffled gives bit-identical outputs.
    kw = dict(batch=4, ctx_lens=[777, 64, 2049, 513], hq=64, hkv=4, d=192, window=window)
    a = make_decode_case(95, shuffle=False, **kw)
    b = make_decode_case(95, shuffle=True, **kw)
    assert not np.array_equal(a.block_table, b.block_table)
    ga = run_decode(a, to_device(a), num_splits=splits).clone()
    gb = run_decode(b, to_device(b), num_splits=splits).clone()
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))
