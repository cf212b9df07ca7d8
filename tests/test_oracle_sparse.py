"""Pins of the Step-5 sparse-attention oracle (oracle/sparse.py) against things
other than itself: torch's bf16 and float8_e4m3fn casts for the two roundings,
closed forms of the coordinatewise block summary, a hand-built weighted-ReLU
score (the ReLU sits inside the sum, weights carry a sign), the selection
rules (ties to the lower id, only blocks before the current one compete, all
candidates when there are at most 512), dense attention when every block is
selected, and a brute-force softmax over the attended tokens otherwise
("Step-5-Preview: Sparse GQA, Indexer und KV-Speicher", the indexer and
attention sections)."""

import numpy as np
import pytest
import torch

from oracle import decode_attention
from oracle.codecs import bf16_bits_to_f64, e4m3fn_codes_to_f64
from oracle.sparse import (attended_tokens, block_summaries, bf16_round, e4m3_round,
                           indexer_scores, select_blocks, sparse_attention)
from workloads import make_decode_case, v_by_subblock


def test_roundings_match_torch_casts():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 1.0, 50.0)])
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).double().numpy())
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(e4m3_round(x.astype(np.float32).astype(np.float64)), ref)


def test_summary_closed_forms():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((16, 256))
    # equal logits: the plain mean of the block's keys
    c, _ = block_summaries(k, np.zeros((16, 256)), 16)
    assert np.allclose(c, k.reshape(2, 8, 256).mean(axis=1), rtol=0, atol=1e-15)
    # one dominant logit per coordinate, a different token per coordinate:
    # each coordinate is that token's coordinate (not any single key vector)
    z = np.full((16, 256), -300.0)
    win = np.arange(256) % 8
    z[win, np.arange(256)] = 300.0
    z[8 + (7 - win), np.arange(256)] = 300.0
    c, codes = block_summaries(k, z, 16)
    assert np.allclose(c[0], k[win, np.arange(256)], rtol=0, atol=1e-12)
    assert np.allclose(c[1], k[8 + 7 - win, np.arange(256)], rtol=0, atol=1e-12)
    # only complete blocks: 15 tokens make one summary, 7 none
    assert block_summaries(k, z, 15)[0].shape == (1, 256)
    assert block_summaries(k, z, 7)[0].shape == (0, 256)
    # storage: E4M3 of the bf16 rounding
    assert np.array_equal(e4m3fn_codes_to_f64(codes), e4m3_round(bf16_round(c)))


def test_score_relu_inside_the_sum_and_signed_weights():
    q = np.zeros((4, 4, 256))
    q[0, 0, 0] = 1.0          # dot with c[0] = +2
    q[0, 1, 1] = 1.0          # dot with c[0] = -3  -> ReLU 0, not -3
    q[1, 0, 0] = 1.0
    w = np.zeros((4, 4))
    w[0, :2] = [1.0, 1.0]
    w[1, 0] = -0.5            # negative weight: negative score
    c = np.zeros((2, 256))
    c[0, 0], c[0, 1] = 2.0, -3.0
    codes = np.stack([np.frombuffer(np.asarray(torch.from_numpy(ci).to(torch.float8_e4m3fn)
                                               .view(torch.uint8).numpy()).tobytes(), np.uint8)
                      for ci in c])
    s = indexer_scores(q, w, codes, t=16)
    assert s.shape == (4, 2)
    assert s[0, 0] == 2.0 and s[1, 0] == -1.0 and s[2, 0] == 0.0
    assert s[0, 1] == 0.0
    # Q8 rounds the query to E4M3 (steps of 1/8 in [1, 2)): 1.07 -> 1.125
    q[0, 0, 0] = 1.07
    assert indexer_scores(q, w, codes, t=16)[0, 0] == 2 * 1.125


def test_selection_rules():
    # ties go to the lower id; ids come back ascending
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert select_blocks(s, budget=2)[0].tolist() == [1, 2]
    assert select_blocks(s, budget=4)[0].tolist() == [1, 2, 3, 4]
    # at most the budget candidates: all of them
    assert select_blocks(np.zeros((1, 7)))[0].tolist() == list(range(7))
    rng = np.random.default_rng(2)
    s = rng.standard_normal((4, 600))
    s[:, 10] = s[:, 11] = np.sort(s[0])[-512]          # a tie straddling the cut of group 0
    sel = select_blocks(s)
    assert all(len(x) == 512 for x in sel)
    thr = np.sort(s[0])[::-1][511]
    assert all(s[0, r] >= thr for r in sel[0])
    # only blocks before the current one compete: t = 8 * 5 + 3 -> five candidates
    assert indexer_scores(np.ones((4, 4, 256)), np.ones((4, 4)),
                          np.full((9, 256), 0x38, np.uint8), t=43).shape == (4, 5)
    # the current block is attended up to t
    assert attended_tokens([0, 2], 43).tolist() == list(range(8)) + list(range(16, 24)) + [40, 41, 42, 43]


def _gqa_case(L, seed=3):
    return make_decode_case(seed, batch=1, ctx_lens=[L], hq=64, hkv=4, d=192, kv_format="bf16",
                            nan_tail=True)


def test_all_blocks_selected_is_dense_attention():
    L = 8 * 300 + 5                     # 300 candidates <= 512: all selected
    case = _gqa_case(L)
    t = L - 1
    sel = [np.arange(t // 8)] * 4
    got = sparse_attention(case.q[0], case.k_cache, v_by_subblock(case.v_cache), case.block_table, 0, t, sel,
                           case.scale)
    ref = decode_attention(case.q, case.k_cache, case.v_cache, [L], case.scale, q_format="bf16",
                           kv_format="bf16", block_table=case.block_table)[0]
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_subset_matches_brute_force_softmax():
    L = 8 * 700 + 2
    case = _gqa_case(L, seed=4)
    t = L - 1
    rng = np.random.default_rng(5)
    sel = [np.sort(rng.choice(t // 8, size=512, replace=False)) for _ in range(4)]
    got = sparse_attention(case.q[0], case.k_cache, v_by_subblock(case.v_cache), case.block_table, 0, t, sel,
                           case.scale)
    for h in (0, 17, 40, 63):
        g = h // 16
        J = [8 * r + e for r in sel[g] for e in range(8)] + list(range(8 * (t // 8), t + 1))
        q = bf16_bits_to_f64(case.q[0, h])
        s, v = [], []
        for j in J:
            blk = case.block_table[0, j // 64]
            s.append(case.scale * bf16_bits_to_f64(case.k_cache[blk, g, j % 64]) @ q)
            v.append(bf16_bits_to_f64(case.v_cache[blk, g, :, j % 64]))
        s = np.array(s)
        p = np.exp(s - s.max())
        want = (p / p.sum()) @ np.array(v)
        assert np.allclose(got[h], want, rtol=0, atol=1e-12), h


# --- the whole decode step (sparse_decode): token position, candidates, composition ---

def _step_batch(lens, seed, nan_tail=True):
    """A Step-5-shaped batch for sparse_decode: paged K, V^T per 8-token
    sub-block, indexer inputs and the summary codes of the complete blocks."""
    from oracle.sparse import sparse_decode  # noqa: F401  (imported by the callers)
    from workloads import make_sparse_indexer_inputs
    case = make_decode_case(seed, batch=len(lens), ctx_lens=lens, hq=64, hkv=4, d=192,
                            kv_format="bf16", nan_tail=nan_tail)
    cap = case.block_table.shape[1] * 64
    idx = make_sparse_indexer_inputs(seed + 1, batch=len(lens), cap=cap)
    codes = np.zeros((len(lens), cap // 8, 256), np.uint8)
    for b, L in enumerate(lens):
        _, c = block_summaries(bf16_bits_to_f64(idx.k_idx[b]), bf16_bits_to_f64(idx.z[b]), L)
        codes[b, :len(c)] = c
    return case, idx, codes


def _bf16_bits(x):
    return np.asarray(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
                      .view(torch.int16).numpy()).view(np.uint16)


def test_step_with_every_candidate_selected_is_dense_attention():
    # t = L - 1 has t // 8 candidate blocks; at most 512 of them (L <= 4104)
    # are all selected, so with the current block the step attends every one
    # of the L keys: dense attention over the whole context.
    from oracle.sparse import sparse_decode
    lens = [1, 7, 8, 9, 65, 1000, 4104, 0]
    case, idx, codes = _step_batch(lens, seed=21)
    out, sels = sparse_decode(case.q, idx.q_idx, idx.w, codes, case.k_cache,
                              v_by_subblock(case.v_cache), case.block_table, case.ctx_lens,
                              case.scale)
    ref = decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                           q_format="bf16", kv_format="bf16", block_table=case.block_table)
    assert np.all(np.isfinite(out))
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    for b, L in enumerate(lens):
        want = np.arange(max(L - 1, 0) // 8)
        assert all(np.array_equal(s, want) for s in sels[b]), b
    assert np.all(out[-1] == 0)                              # L == 0: zeros


@pytest.mark.parametrize("L", [1, 8, 9, 16, 17, 4105, 8 * 600, 8 * 600 + 1])
def test_step_attends_the_token_at_L_minus_1(L):
    # Key L-1 (the decode token's own position) dominates every logit of its
    # group by far more than fp64's exponent range: the step must return its
    # value row exactly.  A step placing the token at L would read the
    # NaN-filled row L; one placing it at L-2 would never attend row L-1.
    from oracle.sparse import sparse_decode
    case, idx, codes = _step_batch([L], seed=22)
    q = np.zeros((1, 64, 192), np.float32)
    q[0, :, 0] = 1.0
    case.q = _bf16_bits(q)
    blk, row = case.block_table[0, (L - 1) // 64], (L - 1) % 64
    case.k_cache[blk, :, row, 0] = _bf16_bits(np.array([3.0e4], np.float32))[0]
    out, _ = sparse_decode(case.q, idx.q_idx, idx.w, codes, case.k_cache,
                           v_by_subblock(case.v_cache), case.block_table, case.ctx_lens,
                           case.scale)
    for g in range(4):
        want = bf16_bits_to_f64(case.v_cache[blk, g, :, row])
        assert np.array_equal(out[0, 16 * g:16 * (g + 1)], np.broadcast_to(want, (16, 192))), g


def test_step_selects_from_the_right_queries_and_candidates():
    # Summaries that are one-hot at coordinate 4b + g for a chosen set of 512
    # blocks of request b and group g, and search queries of request b that
    # are one-hot at those coordinates: each group's selection is its chosen
    # set.  Block (L-1)//8 = t//8 holds the token, so it is no candidate even
    # though its summary scores highest (L = 8k: a token placed at L would
    # make it one).  Reading request 0's queries for request 1 selects
    # request 0's sets instead.
    from oracle.sparse import sparse_attention, sparse_decode
    lens = [8 * 700, 8 * 650]
    case, idx, codes = _step_batch(lens, seed=23, nan_tail=False)
    rng = np.random.default_rng(24)
    codes[:] = 0
    q_idx = np.zeros((2, 4, 4, 256), np.float32)
    w = np.ones((2, 4, 4), np.float32)
    one = 0x38                                               # E4M3 code of 1.0
    chosen = {}
    for b, L in enumerate(lens):
        cand = (L - 1) // 8
        for g in range(4):
            c = 4 * b + g
            q_idx[b, g, :, c] = 1.0
            chosen[b, g] = np.sort(rng.choice(cand, size=512, replace=False))
            codes[b, chosen[b, g], c] = one
            codes[b, cand, c] = 0x7E                          # 448 on the token's own block
    idx.q_idx = _bf16_bits(q_idx)
    out, sels = sparse_decode(case.q, idx.q_idx, w, codes, case.k_cache,
                              v_by_subblock(case.v_cache), case.block_table, case.ctx_lens,
                              case.scale)
    for b, L in enumerate(lens):
        for g in range(4):
            assert np.array_equal(sels[b][g], chosen[b, g]), (b, g)
        ref = sparse_attention(case.q[b], case.k_cache, v_by_subblock(case.v_cache),
                               case.block_table, b, L - 1, [chosen[b, g] for g in range(4)],
                               case.scale)
        assert np.array_equal(out[b], ref)
