"""GPU parity tests of MFA (MQA) decode attention against the fp64 oracle.

All calls go through the C ABI (binding -> libmfa_decode.so).  Sizes are ones
the oracle finishes in seconds while spanning several 64-key tiles, ragged
tails (NaN-filled past each length), empty slots and every split count; the
full-size configurations are checked on every slot.  Bit-exact checks:
block permutation, single key, one-hot logits, repeat runs.
"""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa

from oracle import decode_attention
from workloads import bf16_round_bits, config_case, make_decode_case

from gpu_helpers import assert_parity, run_decode, to_device

pytestmark = pytest.mark.gpu


def oracle(case, slots=None, **over):
    kw = case.oracle_kwargs()
    kw.update(over)
    return decode_attention(case.q, case.k_cache, case.v_cache, kw.pop("ctx_lens", case.ctx_lens),
                            case.scale, slots=slots, **kw)


def test_config1_fp32_contiguous():
    case = config_case(1)
    t = to_device(case)
    got = run_decode(case, t)
    assert_parity(got, oracle(case), "f32", "config 1")


RAGGED = [1, 63, 64, 65, 130, 1000, 0, 4096, 4033]


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_mqa_bf16_paged_ragged(splits):
    case = make_decode_case(101, batch=len(RAGGED), ctx_lens=RAGGED, hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits)
    assert_parity(got, oracle(case), "bf16", f"ragged, splits={splits}")
    assert torch.all(got[6] == 0)          # empty slot


@pytest.mark.parametrize("out_format", ["bf16", "f32"])
def test_more_than_eight_splits(out_format):
    # Twelve forced splits take the running merge over any split count, with
    # bf16 partials (bf16 result) or fp32 ones (fp32 result).
    case = make_decode_case(111, batch=len(RAGGED), ctx_lens=RAGGED, hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case, out_format=out_format)
    got = run_decode(case, t, num_splits=12).clone()
    assert_parity(got, oracle(case), "bf16", f"12 splits, {out_format} out")
    again = run_decode(case, t, num_splits=12)
    assert torch.equal(got, again)


@pytest.mark.parametrize("batch", [7, 8, 13])
@pytest.mark.parametrize("out_format", ["bf16", "f32"])
def test_balanced_partition_grid_sizes(batch, out_format):
    # The balanced cut numbers its workgroups XCD-major when the grid is a
    # multiple of 8 and in launch order otherwise; the merge finds the pieces
    # either way, with bf16 or fp32 partials.
    rng = np.random.default_rng(1000 + batch)
    lens = rng.integers(700, 3000, size=batch).tolist()
    case = make_decode_case(112 + batch, batch=batch, ctx_lens=lens, hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case, out_format=out_format)
    got = run_decode(case, t, num_splits=0)
    assert_parity(got, oracle(case), "bf16", f"balanced, batch {batch}, {out_format} out",
                  per_slot=True)


def test_mqa_bf16_contiguous_cache():
    case = make_decode_case(102, batch=3, ctx_lens=[200, 64, 1], hq=64, hkv=1, d=256,
                            paged=False, scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t)
    assert_parity(got, oracle(case), "bf16", "contiguous")


def test_mqa_fp32_output():
    case = make_decode_case(103, batch=4, ctx_lens=[300, 5, 64, 2000], hq=64, hkv=1, d=256)
    t = to_device(case, out_format="f32")
    got = run_decode(case, t)
    assert got.dtype == torch.float32
    assert_parity(got, oracle(case), "bf16", "fp32 out")


def test_config2_full_size_every_slot():
    # 64 slots x 4096 keys with the heuristic split count: the balanced page
    # cut and the merge the benchmark runs, every slot against the oracle.
    case = config_case(2)
    t = to_device(case)
    got = run_decode(case, t)
    assert_parity(got, oracle(case), "bf16", "config 2", per_slot=True)


def test_config3_ragged_full_size_every_slot():
    # 128 ragged slots: pieces spanning several workgroups, workgroups
    # walking several slots, non-first pieces; every slot against the oracle.
    case = config_case(3)
    t = to_device(case)
    got = run_decode(case, t)
    assert_parity(got, oracle(case), "bf16", "config 3", per_slot=True)


def test_block_permutation_is_bit_exact():
    kw = dict(batch=3, ctx_lens=[777, 64, 2049], hq=64, hkv=1, d=256)
    a = make_decode_case(104, shuffle=False, **kw)
    b = make_decode_case(104, shuffle=True, **kw)
    assert not np.array_equal(a.block_table, b.block_table)
    for splits in (0, 1, 3):
        ga = run_decode(a, to_device(a), num_splits=splits).clone()
        gb = run_decode(b, to_device(b), num_splits=splits).clone()
        assert torch.equal(ga.view(torch.int16), gb.view(torch.int16)), f"splits={splits}"


def test_repeat_runs_are_bit_identical():
    case = make_decode_case(105, batch=8, ctx_lens=[4096, 1, 300, 2500, 64, 65, 999, 3000],
                            hq=64, hkv=1, d=256)
    t = to_device(case)
    first = run_decode(case, t).clone()
    for _ in range(3):
        again = run_decode(case, t)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def _logical_v(case, b, j):
    blk = case.block_table[b, j // 64]
    return case.v_cache[blk, 0, :, j % 64]


def test_single_key_returns_v0_exactly():
    case = make_decode_case(106, batch=3, ctx_lens=[1, 1, 1], hq=64, hkv=1, d=256)
    got = run_decode(case, to_device(case))
    for b in range(3):
        expect = torch.from_numpy(_logical_v(case, b, 0).view(np.int16))
        assert torch.equal(got[b].view(torch.int16).cpu(), expect[None, :].expand(64, -1))


@pytest.mark.parametrize("jstar", [0, 63, 64, 127, 1500, 2999])
def test_one_hot_logits_select_that_value_row_exactly(jstar):
    L = 3000
    case = make_decode_case(107, batch=1, ctx_lens=[L], hq=64, hkv=1, d=256, scale=1 / 16)
    q = np.zeros((1, 64, 256), np.float32)
    q[0, :, 0] = 1.0
    case.q = bf16_round_bits(q)
    blk = case.block_table[0, jstar // 64]
    case.k_cache[blk, 0, jstar % 64, 0] = bf16_round_bits(np.array([2048.0], np.float32))[0]
    for splits in (0, 1, 5):
        got = run_decode(case, to_device(case), num_splits=splits)
        expect = torch.from_numpy(_logical_v(case, 0, jstar).view(np.int16))
        assert torch.equal(got[0].view(torch.int16).cpu(), expect[None, :].expand(64, -1)), splits


def test_length_counts_the_current_token():
    case = make_decode_case(108, batch=1, ctx_lens=[1000], hq=64, hkv=1, d=256)
    t = to_device(case)
    full = run_decode(case, t).clone()
    shorter = run_decode(case, t, lens=torch.tensor([999], dtype=torch.int32, device="cuda"))
    assert not torch.equal(full, shorter)
    assert_parity(shorter, oracle(case, ctx_lens=np.array([999])), "bf16", "L-1")


def test_balanced_partition_many_short_slots():
    # Heuristic split count on a paged MQA batch: the workgroups divide the
    # batch's actual pages, so one workgroup walks several short slots and
    # long slots span several workgroups; empty slots sit in between.
    lens = [1, 0, 63, 64, 65, 0, 130, 4096, 1, 2, 700, 0, 4033, 128, 129, 5, 3000, 64] * 2
    case = make_decode_case(109, batch=len(lens), ctx_lens=lens, hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t, num_splits=0).clone()
    assert_parity(got, oracle(case), "bf16", "balanced partition")
    for b in np.flatnonzero(np.array(lens) == 0):
        assert torch.all(got[b] == 0)
    again = run_decode(case, t, num_splits=0)
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("length", [3000, 4033, 64])
def test_balanced_partition_uniform_lengths(length):
    # Every slot the same length below the table capacity: the kernel's
    # predicted cut (from one slot's length) is the real one.
    case = make_decode_case(110, batch=24, ctx_lens=[length] * 24, hq=64, hkv=1, d=256,
                            scale=1 / 16, table_width=64)
    t = to_device(case)
    got = run_decode(case, t, num_splits=0).clone()
    assert_parity(got, oracle(case), "bf16", f"uniform {length}")
    again = run_decode(case, t, num_splits=0)
    assert torch.equal(got.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_two_phases_equal_the_whole_call(splits):
    # mfa_decode_attention_phase 1 (attention) then 2 (merge) is the same
    # computation as mfa_decode_attention: bit-identical outputs.
    case = make_decode_case(331, batch=6, ctx_lens=[1, 64, 700, 4096, 0, 2049], hq=64, hkv=1,
                            d=256, scale=1 / 16)
    t = to_device(case)
    whole = torch.full_like(t["out"], float("nan"))
    mfa.mfa_decode_attention(t["q"], t["k"], t["v"], t["table"], t["lens"], whole, case.scale,
                             num_splits=splits)
    phased = torch.full_like(t["out"], float("nan"))
    for phase in (1, 2):
        mfa.mfa_decode_attention_phase(t["q"], t["k"], t["v"], t["table"], t["lens"], phased,
                                       case.scale, phase, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), phased.view(torch.int16))
