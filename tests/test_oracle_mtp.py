"""Pins of the multi-token decode oracle (oracle/mtp.py) against things other
than itself: a brute-force masked [Tq x L] softmax with its own block-table
walk (the causal mask written as "key position <= the token's position"), the
closed form q = 0 (each token returns the mean of V over its own prefix), the
causality invariant (keys after token t do not move token t but do move token
t + 1), and Tq = 1 reducing to single-token decode.  Reading pinned: the Tq
new tokens are the last Tq cached keys and token t attends the first
L - (Tq - 1 - t) of them ("Step-3 is Large yet Affordable", section 5.2)."""

import numpy as np
import pytest

from oracle import decode_attention, decode_attention_mtp, mtp_lengths
from workloads import make_decode_case, make_mtp_queries

PAGE = 64


def _case(lens, *, kv_format="f32", hq=4, d=8, seed=3, paged=True):
    return make_decode_case(seed, batch=len(lens), ctx_lens=lens, hq=hq, hkv=1, d=d,
                            kv_format=kv_format, scale=0.3, paged=paged, nan_tail=False)


def _brute(case, q, lens):
    """Masked softmax over the whole [Tq, L] score matrix of each sequence and
    head, f32 storage read directly (no codecs), keys gathered one by one."""
    B, tq, hq, d = q.shape
    out = np.zeros((B, tq, hq, d))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        K = np.array([case.k_cache[case.block_table[b, j // PAGE], 0, j % PAGE, :] for j in range(L)],
                     dtype=np.float64)
        V = np.array([case.v_cache[case.block_table[b, j // PAGE], 0, :, j % PAGE] for j in range(L)],
                     dtype=np.float64)
        pos = L - tq + np.arange(tq)                       # absolute position of each new token
        allowed = np.arange(L)[None, :] <= pos[:, None]    # [Tq, L]
        for h in range(hq):
            S = case.scale * (q[b, :, h, :].astype(np.float64) @ K.T)
            S = np.where(allowed, S, -np.inf)
            for t in range(tq):
                if not allowed[t].any():
                    continue
                e = np.exp(S[t] - S[t].max())
                out[b, t, h] = (e / e.sum()) @ V
    return out


def test_lengths_of_each_token():
    assert mtp_lengths([10, 2, 0], 3).tolist() == [[8, 9, 10], [0, 1, 2], [0, 0, 0]]
    assert mtp_lengths([7], 1).tolist() == [[7]]


@pytest.mark.parametrize("tq", [1, 2, 3, 5])
def test_matches_brute_force_masked_softmax(tq):
    lens = np.array([70, 2, 64, 129], dtype=np.int64)
    case = _case(lens)
    q = make_mtp_queries(5, batch=len(lens), tq=tq, hq=4, d=8, q_format="f32")
    got = decode_attention_mtp(q, case.k_cache, case.v_cache, lens, case.scale,
                               q_format="f32", kv_format="f32", block_table=case.block_table)
    assert np.allclose(got, _brute(case, q, lens), rtol=0, atol=1e-12)


def test_zero_query_gives_each_token_its_prefix_mean():
    lens = np.array([65, 3, 130], dtype=np.int64)
    tq = 4
    case = _case(lens)
    q = np.zeros((len(lens), tq, 4, 8), np.float32)
    got = decode_attention_mtp(q, case.k_cache, case.v_cache, lens, case.scale,
                               q_format="f32", kv_format="f32", block_table=case.block_table)
    for b, L in enumerate(lens):
        V = np.array([case.v_cache[case.block_table[b, j // PAGE], 0, :, j % PAGE] for j in range(L)],
                     dtype=np.float64)
        for t in range(tq):
            n = L - (tq - 1 - t)
            want = V[:n].mean(axis=0) if n > 0 else np.zeros(8)
            assert np.allclose(got[b, t], want[None, :], rtol=0, atol=1e-12), (b, t)


def test_keys_after_a_token_do_not_move_it():
    lens = np.array([100, 64], dtype=np.int64)
    tq = 3
    case = _case(lens)
    q = make_mtp_queries(9, batch=2, tq=tq, hq=4, d=8, q_format="f32")
    kw = dict(q_format="f32", kv_format="f32", block_table=case.block_table)
    base = decode_attention_mtp(q, case.k_cache, case.v_cache, lens, case.scale, **kw)
    for t in range(tq - 1):
        k2, v2 = case.k_cache.copy(), case.v_cache.copy()
        for b, L in enumerate(lens):
            for j in range(L - (tq - 1 - t), L):           # the keys after token t
                blk = case.block_table[b, j // PAGE]
                k2[blk, 0, j % PAGE, :] += 3.0
                v2[blk, 0, :, j % PAGE] -= 5.0
        moved = decode_attention_mtp(q, k2, v2, lens, case.scale, **kw)
        assert np.array_equal(moved[:, :t + 1], base[:, :t + 1])
        assert not np.allclose(moved[:, t + 1], base[:, t + 1])


def test_single_token_is_plain_decode():
    lens = np.array([1, 63, 64, 300], dtype=np.int64)
    case = _case(lens, kv_format="bf16", hq=8, d=16)
    q = make_mtp_queries(11, batch=4, tq=1, hq=8, d=16, q_format="bf16")
    kw = dict(q_format="bf16", kv_format="bf16", block_table=case.block_table)
    got = decode_attention_mtp(q, case.k_cache, case.v_cache, lens, case.scale, **kw)
    ref = decode_attention(q[:, 0], case.k_cache, case.v_cache, lens, case.scale, **kw)
    assert np.array_equal(got[:, 0], ref)
