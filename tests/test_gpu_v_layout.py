"""GPU tests of the second V layout (8-token sub-blocks, the sparse global
attention's layout) on the dense per-group entry and the KV append, and of the
incremental block summaries: one cache of the Step-5 global layer serves the
dense call, the sparse call and the append ("Step-5-Preview: Sparse GQA,
Indexer und KV-Speicher": the sparse path attends to the original K/V; a
block is summarised when its eighth token arrives).

The sub-blocked V holds the same values as the channel-major one, so the
dense results must be bit-identical between the two layouts, and both within
the bf16 bar of the fp64 oracle."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention, kv_append
from oracle.codecs import bf16_bits_to_f64
from oracle.sparse import block_summaries
from workloads import bf16_round_bits, make_decode_case, make_sparse_indexer_inputs, v_by_subblock

from gpu_helpers import _raw_to_tensor, assert_parity, to_device

pytestmark = pytest.mark.gpu

LENS = [1, 63, 511, 512, 513, 700, 2000, 0]


def _bits16(t):
    return t.detach().cpu().view(torch.int16).numpy()


def _dense(case, t, v, window, splits, v_layout):
    out = torch.full((case.batch, case.hq, case.d), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    mfa.mfa_decode_attention_gqa(t["q"], t["k"], v, t["table"], t["lens"], out, case.scale,
                                 window=window, num_splits=splits, v_layout=v_layout)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("window", [0, 512, 100])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_dense_call_reads_sub_blocked_v_bit_identically(paged, window, splits):
    print(f"v layout: paged={paged} window={window} splits={splits}", flush=True)
    case = make_decode_case(80 + window, batch=len(LENS), ctx_lens=LENS, hq=64, hkv=4, d=192,
                            window=window, paged=paged)
    t = to_device(case)
    v_sub = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
    a = _dense(case, t, t["v"], window, splits, "channel")
    b = _dense(case, t, v_sub, window, splits, "subblock8")
    assert np.array_equal(_bits16(a), _bits16(b))
    ref = decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                           **case.oracle_kwargs())
    assert_parity(b, ref, "bf16", f"sub-blocked V window={window} splits={splits}")


def test_width_256_groups_read_sub_blocked_v():
    case = make_decode_case(88, batch=4, ctx_lens=[65, 1000, 0, 257], hq=32, hkv=2, d=256,
                            scale=1 / 16)
    t = to_device(case)
    v_sub = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
    a = _dense(case, t, t["v"], 0, 2, "channel")
    b = _dense(case, t, v_sub, 0, 2, "subblock8")
    assert np.array_equal(_bits16(a), _bits16(b))


@pytest.mark.parametrize("paged", [True, False])
def test_append_writes_sub_blocked_v_bit_for_bit(paged):
    lens = np.array([0, 1, 7, 8, 63, 64, 65, 200], dtype=np.int64)
    case = make_decode_case(89, batch=len(lens), ctx_lens=lens + 1, hq=64, hkv=4, d=192,
                            paged=paged)
    rng = np.random.default_rng(90)
    k_new = bf16_round_bits(rng.standard_normal((len(lens), 4, 192), dtype=np.float32))
    v_new = bf16_round_bits(rng.standard_normal((len(lens), 4, 192), dtype=np.float32))
    t = to_device(case)
    v_sub = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
    dlens = torch.from_numpy(lens.astype(np.int32)).cuda()
    mfa.mfa_kv_append(_raw_to_tensor(k_new, "bf16", "cuda"), _raw_to_tensor(v_new, "bf16", "cuda"),
                      t["k"], v_sub, t["table"], dlens, v_layout="subblock8")
    torch.cuda.synchronize()
    rk, rv, rl = kv_append(case.k_cache, case.v_cache, lens, k_new, v_new, new_format="bf16",
                           kv_format="bf16", block_table=case.block_table)
    assert np.array_equal(dlens.cpu().numpy().astype(np.int64), rl)
    assert np.array_equal(t["k"].cpu().view(torch.int16).numpy().view(np.uint16), rk)
    assert np.array_equal(v_sub.cpu().view(torch.int16).numpy().view(np.uint16),
                          v_by_subblock(rv))


def _summaries_host(idx, lens, cap8, fill):
    codes = np.full((len(lens), cap8, 256), fill, np.uint8)
    for b, L in enumerate(lens):
        _, c = block_summaries(bf16_bits_to_f64(idx.k_idx[b]), bf16_bits_to_f64(idx.z[b]), int(L))
        codes[b, :len(c)] = c
    return codes


def test_incremental_summaries_equal_a_full_pass():
    """Start from the full summaries at L0, then advance the lengths by n
    tokens at a time and summarise only the blocks those tokens completed:
    after every call the array equals a fresh full pass at the new lengths,
    and entries past the complete blocks keep their sentinel."""
    L0 = np.array([0, 5, 8, 15, 16, 63, 100, 4095], dtype=np.int64)
    cap = 4224
    table = torch.zeros((len(L0), cap // 64), dtype=torch.int32, device="cuda")
    idx = make_sparse_indexer_inputs(91, batch=len(L0), cap=cap)
    k_idx = _raw_to_tensor(idx.k_idx, "bf16", "cuda")
    z = _raw_to_tensor(idx.z, "bf16", "cuda")
    cap8 = cap // 8
    summ = torch.full((len(L0), cap8, 256), 0x5A, dtype=torch.uint8, device="cuda")
    lens = L0.copy()
    dlens = torch.from_numpy(lens.astype(np.int32)).cuda()
    mfa.mfa_sparse_summarize(k_idx, z, dlens, summ, block_table=table)
    for n in [1] * 17 + [8, 13, 3, 64]:
        lens = lens + n
        dlens.copy_(torch.from_numpy(lens.astype(np.int32)))
        mfa.mfa_sparse_summarize_new(k_idx, z, dlens, summ, n, block_table=table)
        full = torch.full_like(summ, 0x5A)
        mfa.mfa_sparse_summarize(k_idx, z, dlens, full, block_table=table)
        torch.cuda.synchronize()
        assert torch.equal(summ, full), (n, lens)
    # The final state against the oracle: the complete blocks hold codes within
    # the summaries' own bar (at most 1 % one E4M3 step off), the rest keeps
    # the sentinel.
    ref = _summaries_host(idx, lens, cap8, 0x5A)
    got = summ.cpu().numpy()
    for b, L in enumerate(lens):
        nb = int(L) // 8
        assert np.all(got[b, nb:] == 0x5A), b
        assert (got[b, :nb] != ref[b, :nb]).mean() < 0.01, b


def test_one_cache_serves_dense_sparse_and_append():
    """A Step-5 global-layer cache with V in sub-blocks: append a token, then
    run the dense per-group call and the whole sparse step (summaries,
    selection, attention) on the same K/V.  At L <= 4104 every candidate block
    is selected, so both equal the dense attention over all L keys."""
    lens0 = np.array([299, 4000, 1, 4103], dtype=np.int64)
    case = make_decode_case(92, batch=len(lens0), ctx_lens=lens0 + 1, hq=64, hkv=4, d=192)
    idx = make_sparse_indexer_inputs(93, batch=len(lens0), cap=case.max_blocks * 64)
    t = to_device(case)
    v_sub = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
    rng = np.random.default_rng(94)
    k_new = bf16_round_bits(rng.standard_normal((len(lens0), 4, 192), dtype=np.float32))
    v_new = bf16_round_bits(rng.standard_normal((len(lens0), 4, 192), dtype=np.float32))
    dlens = torch.from_numpy(lens0.astype(np.int32)).cuda()
    mfa.mfa_kv_append(_raw_to_tensor(k_new, "bf16", "cuda"), _raw_to_tensor(v_new, "bf16", "cuda"),
                      t["k"], v_sub, t["table"], dlens, v_layout="subblock8")
    rk, rv, rl = kv_append(case.k_cache, case.v_cache, lens0, k_new, v_new, new_format="bf16",
                           kv_format="bf16", block_table=case.block_table)
    ref = decode_attention(case.q, rk, rv, rl, case.scale, **case.oracle_kwargs())

    dense = torch.full((case.batch, 64, 192), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_decode_attention_gqa(t["q"], t["k"], v_sub, t["table"], dlens, dense, case.scale,
                                 v_layout="subblock8")
    k_idx = _raw_to_tensor(idx.k_idx, "bf16", "cuda")
    z = _raw_to_tensor(idx.z, "bf16", "cuda")
    summ = torch.zeros((case.batch, case.max_blocks * 8, 256), dtype=torch.uint8, device="cuda")
    sel = torch.full((case.batch, 4, 512), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((case.batch, 4), -7, dtype=torch.int32, device="cuda")
    sparse = torch.full_like(dense, float("nan"))
    mfa.mfa_sparse_summarize(k_idx, z, dlens, summ, block_table=t["table"])
    mfa.mfa_sparse_select(_raw_to_tensor(idx.q_idx, "bf16", "cuda"), torch.from_numpy(idx.w).cuda(),
                          summ, dlens, sel, nsel, block_table=t["table"])
    mfa.mfa_sparse_attention(t["q"], t["k"], v_sub, t["table"], dlens, sel, nsel, sparse,
                             case.scale)
    torch.cuda.synchronize()
    assert np.array_equal(nsel.cpu().numpy(), np.repeat(((rl - 1) // 8)[:, None], 4, axis=1))
    assert_parity(dense, ref, "bf16", "dense call on the shared cache")
    assert_parity(sparse, ref, "bf16", "sparse call on the shared cache")
