"""The allocation-free decode entry (mfa_decode_attention_noalloc) against the
workspace entry it varies (mfa_decode_attention): same kernels, so the outputs
must agree bit for bit, and both stay within the oracle's tolerance.  Two
calls in a row share the library's scratch array, the second on a smaller
batch; a call needing more than the array is refused on the host."""

import ctypes

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from decode_attention_mfa_amd import _lib
from oracle import decode_attention
from workloads import make_decode_case

from gpu_helpers import assert_parity, to_device

pytestmark = pytest.mark.gpu


def _both(case, num_splits=0):
    t = to_device(case)
    ref_out = torch.full_like(t["out"], float("nan"))
    mfa.mfa_decode_attention(t["q"], t["k"], t["v"], t["table"], t["lens"], ref_out, case.scale,
                             k_scale=t["k_scale"], v_scale=t["v_scale"], num_splits=num_splits)
    got = torch.full_like(t["out"], float("nan"))
    mfa.mfa_decode_attention_noalloc(t["q"], t["k"], t["v"], t["table"], t["lens"], got,
                                     case.scale, k_scale=t["k_scale"], v_scale=t["v_scale"],
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return got, ref_out


def test_two_calls_in_a_row_match_the_workspace_entry():
    # First a full-size call (the balanced page cut of 64 slots x 4096 keys,
    # 32 MB of partials), then a smaller ragged batch: the second call reuses
    # the array the first one left filled.
    big = make_decode_case(301, batch=64, ctx_lens=[4096] * 64, hq=64, hkv=1, d=256,
                           scale=1 / 16)
    small = make_decode_case(302, batch=9, ctx_lens=[1, 63, 64, 65, 130, 1000, 0, 4096, 4033],
                             hq=64, hkv=1, d=256, scale=1 / 16)
    for case in (big, small):
        got, ref_out = _both(case)
        assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), case.batch
        ref = decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                               **case.oracle_kwargs())
        assert_parity(got, ref, "bf16", f"noalloc B={case.batch}", per_slot=True)
    # forced splits and an FP8 cache take the same array
    fp8 = make_decode_case(303, batch=5, ctx_lens=[5, 640, 0, 1111, 3000], hq=64, hkv=1, d=256,
                           kv_format="e4m3", scale=1 / 16)
    got, ref_out = _both(fp8, num_splits=3)
    assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16))


def test_calls_needing_more_than_the_array_are_refused():
    lib = _lib.load()
    d = _lib.MfaDecodeDesc(batch=4096, num_q_heads=64, num_kv_heads=1, head_dim=256, page_size=64,
                           max_blocks_per_seq=64, num_blocks=4096 * 64, q_dtype=_lib.MFA_BF16,
                           kv_dtype=_lib.MFA_BF16, out_dtype=_lib.MFA_BF16, num_splits=8)
    assert lib.mfa_decode_workspace_size(ctypes.byref(d), 0) > 64 << 20
    a = ctypes.c_void_p(0x10000)
    assert lib.mfa_decode_attention_noalloc(ctypes.byref(d), a, a, a, a, a, None, None, a,
                                            ctypes.c_float(0.0625), None) == 6   # MFA_ERR_WORKSPACE
