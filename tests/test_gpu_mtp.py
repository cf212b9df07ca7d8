"""GPU parity of multi-token decode queries (mfa_decode_attention_mtp) against
the oracle: Tq new tokens per sequence, causal among themselves ("Step-3 is
Large yet Affordable", section 5.2, MTP).  Ragged lengths include sequences
shorter than Tq (tokens with no key get zeros), page boundaries and the Step-3
shape (B=64, L=4096, Tq=2) in the launch configuration the bench times."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention_mtp
from workloads import make_decode_case, make_mtp_queries

from gpu_helpers import _raw_to_tensor, assert_parity, to_device

pytestmark = pytest.mark.gpu

LENS = [0, 1, 2, 3, 63, 64, 65, 200, 1000, 2049]


def _run(case, q_raw, tq, *, num_splits=0, out_f32=False):
    t = to_device(case)
    q = _raw_to_tensor(q_raw, case.q_format, "cuda")
    odt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((case.batch, tq, case.hq, case.d), float("nan"), dtype=odt, device="cuda")
    mfa.mfa_decode_attention_mtp(q, t["k"], t["v"], t["table"], t["lens"], out, case.scale,
                                 k_scale=t["k_scale"], v_scale=t["v_scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return out, t


def _ref(case, q_raw, slots=None):
    return decode_attention_mtp(q_raw, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                                q_format=case.q_format, kv_format=case.kv_format,
                                block_table=case.block_table, k_scale=case.k_scale,
                                v_scale=case.v_scale, slots=slots)


@pytest.mark.parametrize("kv_format", ["bf16", "e4m3"])
@pytest.mark.parametrize("tq", [2, 3, 4])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mtp_matches_oracle(kv_format, tq, splits):
    case = make_decode_case(61 + tq, batch=len(LENS), ctx_lens=LENS, kv_format=kv_format)
    q = make_mtp_queries(71 + tq, batch=len(LENS), tq=tq)
    out, _ = _run(case, q, tq, num_splits=splits)
    ref = _ref(case, q)
    assert_parity(out, ref, kv_format, f"mtp {kv_format} tq={tq} splits={splits}")
    # tokens with no key left are exactly zero
    for b, L in enumerate(LENS):
        for t in range(tq):
            if L - (tq - 1 - t) <= 0:
                assert torch.count_nonzero(out[b, t]) == 0, (b, t)


def test_single_token_is_the_plain_call_bit_for_bit():
    case = make_decode_case(81, batch=len(LENS), ctx_lens=LENS, kv_format="bf16")
    q = make_mtp_queries(82, batch=len(LENS), tq=1)
    out, t = _run(case, q, 1)
    plain = torch.full_like(out[:, 0], float("nan"))
    mfa.mfa_decode_attention(_raw_to_tensor(q[:, 0], "bf16", "cuda"), t["k"], t["v"], t["table"],
                             t["lens"], plain, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0].view(torch.int16), plain.view(torch.int16))


def test_sixteen_tokens_and_f32_output():
    lens = [5, 16, 17, 64, 300]
    case = make_decode_case(83, batch=len(lens), ctx_lens=lens, kv_format="bf16")
    q = make_mtp_queries(84, batch=len(lens), tq=16)
    out, _ = _run(case, q, 16, out_f32=True)
    assert_parity(out, _ref(case, q), "bf16", "mtp tq=16")


def test_contiguous_cache():
    case = make_decode_case(85, batch=len(LENS), ctx_lens=LENS, kv_format="bf16", paged=False)
    q = make_mtp_queries(86, batch=len(LENS), tq=2)
    out, _ = _run(case, q, 2, num_splits=2)
    assert_parity(out, _ref(case, q), "bf16", "mtp contiguous")


def test_step3_shape_two_tokens_every_slot():
    # B=64 sequences of 4096 keys, two new tokens each (MTP with one draft),
    # heuristic splits as the bench runs it; every sequence vs the oracle.
    case = make_decode_case(87, batch=64, ctx_lens=[4096] * 64, kv_format="bf16")
    q = make_mtp_queries(88, batch=64, tq=2)
    out, _ = _run(case, q, 2)
    assert_parity(out, _ref(case, q), "bf16", "mtp B=64 L=4096 Tq=2", per_slot=True)
