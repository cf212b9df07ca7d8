"""GPU parity of the Step-5 sparse global attention ("Step-5-Preview: Sparse
GQA, Indexer und KV-Speicher", indexer and attention sections) against the
oracle: block summaries (each code the oracle's, or one E4M3 step from the
exact value where fp32 and fp64 round differently), the top-512 selection
(identical, or differing only between blocks whose scores tie with the cut
to fp32 precision; exact ties go to the lower id), and attention over the
selected blocks plus the current block (within the bf16 bar)."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle.codecs import bf16_bits_to_f64, e4m3fn_codes_to_f64
from oracle.sparse import (block_summaries, indexer_scores, select_blocks, sparse_attention,
                           sparse_decode)
from workloads import make_decode_case, make_sparse_indexer_inputs, v_by_subblock

from gpu_helpers import _raw_to_tensor, assert_parity

pytestmark = pytest.mark.gpu

LENS = [1, 8, 9, 100, 4100, 4105, 9001, 20000]


def _case(lens, seed=31):
    case = make_decode_case(seed, batch=len(lens), ctx_lens=lens, hq=64, hkv=4, d=192,
                            kv_format="bf16", nan_tail=True)
    idx = make_sparse_indexer_inputs(seed + 1, batch=len(lens), cap=case.max_blocks * 64)
    return case, idx


def _host_summaries(case, idx):
    cap8 = case.max_blocks * 8
    codes = np.zeros((case.batch, cap8, 256), np.uint8)
    for b, L in enumerate(case.ctx_lens):
        _, c = block_summaries(bf16_bits_to_f64(idx.k_idx[b]), bf16_bits_to_f64(idx.z[b]), int(L))
        codes[b, :len(c)] = c
    return codes


def _dev(case, idx, summ):
    return dict(
        table=torch.from_numpy(case.block_table).cuda(),
        lens=torch.from_numpy(case.ctx_lens.astype(np.int32)).cuda(),
        q_idx=_raw_to_tensor(idx.q_idx, "bf16", "cuda"),
        w=torch.from_numpy(idx.w).cuda(),
        k_idx=_raw_to_tensor(idx.k_idx, "bf16", "cuda"),
        z=_raw_to_tensor(idx.z, "bf16", "cuda"),
        summ=torch.from_numpy(summ).cuda(),
        sel=torch.full((case.batch, 4, 512), -7, dtype=torch.int32, device="cuda"),
        nsel=torch.full((case.batch, 4), -7, dtype=torch.int32, device="cuda"),
    )


def test_summaries():
    case, idx = _case(LENS)
    ref = _host_summaries(case, idx)
    d = _dev(case, idx, np.full_like(ref, 0x5A))
    mfa.mfa_sparse_summarize(d["k_idx"], d["z"], d["lens"], d["summ"], block_table=d["table"])
    got = d["summ"].cpu().numpy()
    for b, L in enumerate(case.ctx_lens):
        nb = int(L) // 8
        assert np.all(got[b, nb:] == 0x5A)                   # incomplete / absent blocks untouched
        if nb == 0:
            continue
        exact, _ = block_summaries(bf16_bits_to_f64(idx.k_idx[b]), bf16_bits_to_f64(idx.z[b]), int(L))
        g, r = got[b, :nb], ref[b, :nb]
        diff = g != r
        assert diff.mean() < 0.01, diff.mean()
        # a differing code is the other neighbour of the exact value (one step away)
        gv, rv = e4m3fn_codes_to_f64(g[diff]), e4m3fn_codes_to_f64(r[diff])
        ex = exact[diff]
        assert np.all((np.minimum(gv, rv) <= ex + 1e-3 * np.abs(ex)) &
                      (np.maximum(gv, rv) >= ex - 1e-3 * np.abs(ex)))


def _ref_selection(case, idx, summ):
    out = []
    for b, L in enumerate(case.ctx_lens):
        t = int(L) - 1
        s = indexer_scores(bf16_bits_to_f64(idx.q_idx[b]), idx.w[b], summ[b], t)
        out.append((s, select_blocks(s)))
    return out


def test_selection():
    case, idx = _case(LENS)
    summ = _host_summaries(case, idx)
    d = _dev(case, idx, summ)
    mfa.mfa_sparse_select(d["q_idx"], d["w"], d["summ"], d["lens"], d["sel"], d["nsel"],
                          block_table=d["table"])
    sel, nsel = d["sel"].cpu().numpy(), d["nsel"].cpu().numpy()
    for b, (s, ref) in enumerate(_ref_selection(case, idx, summ)):
        for g in range(4):
            n = len(ref[g])
            assert nsel[b, g] == n
            got = sel[b, g, :n]
            assert np.all(np.diff(got) > 0)                  # ascending ids
            if np.array_equal(got, ref[g]):
                continue
            # only near-ties with the 512th score may swap
            thr = np.sort(s[g])[::-1][511]
            swapped = np.setxor1d(got, ref[g])
            assert np.all(np.abs(s[g][swapped] - thr) <= 1e-5 * (1 + abs(thr))), (b, g)


def test_exact_ties_go_to_the_lower_block():
    # Every block of a request gets the same summary: all scores are equal,
    # and the first 512 candidates are selected.
    case, idx = _case([8 * 900 + 3, 8 * 513 + 7])
    summ = _host_summaries(case, idx)
    summ[:, 1:] = summ[:, :1]
    d = _dev(case, idx, summ)
    mfa.mfa_sparse_select(d["q_idx"], d["w"], d["summ"], d["lens"], d["sel"], d["nsel"],
                          block_table=d["table"])
    assert np.array_equal(d["sel"].cpu().numpy(), np.broadcast_to(np.arange(512), (2, 4, 512)))


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_attention_over_the_oracle_selection(splits):
    case, idx = _case(LENS)
    summ = _host_summaries(case, idx)
    refsel = _ref_selection(case, idx, summ)
    d = _dev(case, idx, summ)
    sel = np.zeros((case.batch, 4, 512), np.int32)
    nsel = np.zeros((case.batch, 4), np.int32)
    for b, (_, ref) in enumerate(refsel):
        for g in range(4):
            sel[b, g, :len(ref[g])] = ref[g]
            nsel[b, g] = len(ref[g])
    q = _raw_to_tensor(case.q, "bf16", "cuda")
    k = _raw_to_tensor(case.k_cache, "bf16", "cuda")
    vs = v_by_subblock(case.v_cache)                    # this layer's V layout
    v = _raw_to_tensor(vs, "bf16", "cuda")
    out = torch.full((case.batch, 64, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_sparse_attention(q, k, v, d["table"], d["lens"], torch.from_numpy(sel).cuda(),
                             torch.from_numpy(nsel).cuda(), out, case.scale, num_splits=splits)
    torch.cuda.synchronize()
    ref = np.stack([sparse_attention(case.q[b], case.k_cache, vs, case.block_table, b,
                                     int(L) - 1, refsel[b][1], case.scale)
                    for b, L in enumerate(case.ctx_lens)])
    assert_parity(out, ref, "bf16", f"sparse attention splits={splits}")


def test_whole_step_end_to_end():
    # Equal compression logits make the summaries exact in fp32 (the mean of
    # 8 bf16 values), so both sides select from identical codes; random logits
    # are covered by test_summaries.
    lens = [4105, 12000, 300, 32768]
    case, idx = _case(lens, seed=41)
    idx.z[:] = 0
    d = _dev(case, idx, np.zeros((case.batch, case.max_blocks * 8, 256), np.uint8))
    q = _raw_to_tensor(case.q, "bf16", "cuda")
    k = _raw_to_tensor(case.k_cache, "bf16", "cuda")
    vs = v_by_subblock(case.v_cache)                    # this layer's V layout
    v = _raw_to_tensor(vs, "bf16", "cuda")
    out = torch.empty((case.batch, 64, 192), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_sparse_summarize(d["k_idx"], d["z"], d["lens"], d["summ"], block_table=d["table"])
    mfa.mfa_sparse_select(d["q_idx"], d["w"], d["summ"], d["lens"], d["sel"], d["nsel"],
                          block_table=d["table"])
    mfa.mfa_sparse_attention(q, k, v, d["table"], d["lens"], d["sel"], d["nsel"], out, case.scale)
    torch.cuda.synchronize()
    summ = _host_summaries(case, idx)
    assert np.array_equal(d["summ"].cpu().numpy(), summ)
    ref, refsel = sparse_decode(case.q, idx.q_idx, idx.w, summ, case.k_cache, vs,
                                case.block_table, case.ctx_lens, case.scale)
    gsel, gn = d["sel"].cpu().numpy(), d["nsel"].cpu().numpy()
    for b in range(case.batch):
        for g in range(4):
            assert np.array_equal(gsel[b, g, :gn[b, g]], refsel[b][g]), (b, g)
    assert_parity(out, ref, "bf16", "sparse step end to end")


def test_bad_selections_are_clamped_into_the_candidates():
    # Ids below 0 or past the candidates and counts outside [0, 512] are the
    # caller's error; the kernel clamps them (id -> [0, R - 1], count ->
    # [0, min(R, 512)]) and so reads only the request's own blocks.
    case, idx = _case([4105, 300, 9])
    R = [(int(L) - 1) // 8 for L in case.ctx_lens]
    rng = np.random.default_rng(5)
    sel = rng.integers(-50, 1000, size=(3, 4, 512)).astype(np.int32)
    nsel = np.array([[600, 512, -3, 100], [40, 37, 1000, 0], [5, 0, 1, -1]], np.int32)
    vs = v_by_subblock(case.v_cache)
    q = _raw_to_tensor(case.q, "bf16", "cuda")
    out = torch.full((3, 64, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_sparse_attention(q, _raw_to_tensor(case.k_cache, "bf16", "cuda"),
                             _raw_to_tensor(vs, "bf16", "cuda"),
                             torch.from_numpy(case.block_table).cuda(),
                             torch.from_numpy(case.ctx_lens.astype(np.int32)).cuda(),
                             torch.from_numpy(sel).cuda(), torch.from_numpy(nsel).cuda(), out,
                             case.scale)
    torch.cuda.synchronize()
    ref = []
    for b, L in enumerate(case.ctx_lens):
        n = np.clip(nsel[b], 0, min(R[b], 512))
        clamped = [np.clip(sel[b, g, :n[g]], 0, max(R[b] - 1, 0)) for g in range(4)]
        ref.append(sparse_attention(case.q[b], case.k_cache, vs, case.block_table, b, int(L) - 1,
                                    clamped, case.scale))
    assert_parity(out, np.stack(ref), "bf16", "clamped selections")
