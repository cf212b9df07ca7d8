"""A captured decode loop on one Step-5 global-layer cache ("Step-5-Preview:
Sparse GQA, Indexer und KV-Speicher"): each step appends the new token's K/V
into the cache with V in 8-token sub-blocks, summarises the block that token
completes (a block is summarised at its eighth token), scores and selects the
top-512 blocks, attends over the selection, and runs the dense per-group call
on the same cache.  The step is captured once in a HIP graph and replayed
with the lengths advancing on the device; every replay is checked bit for bit
against the same step run eagerly on a copy of the state, and the last one
against the oracle (at L <= 4104 every candidate is selected, so the sparse
and the dense result both equal dense attention over all L keys)."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention, kv_append
from workloads import bf16_round_bits, make_decode_case, make_sparse_indexer_inputs, v_by_subblock

from gpu_helpers import _raw_to_tensor, assert_parity, to_device

pytestmark = pytest.mark.gpu

STEPS = 9


def test_captured_step5_loop_replays_like_eager():
    lens0 = np.array([7, 100, 3990, 1], dtype=np.int64)
    case = make_decode_case(180, batch=len(lens0), ctx_lens=lens0 + STEPS, hq=64, hkv=4, d=192)
    idx = make_sparse_indexer_inputs(181, batch=len(lens0), cap=case.max_blocks * 64)
    rng = np.random.default_rng(182)
    news = [(bf16_round_bits(rng.standard_normal((len(lens0), 4, 192), dtype=np.float32)),
             bf16_round_bits(rng.standard_normal((len(lens0), 4, 192), dtype=np.float32)))
            for _ in range(STEPS)]

    def state():
        t = to_device(case)
        t["v"] = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
        t["lens"] = torch.from_numpy(lens0.astype(np.int32)).cuda()
        t["kn"] = torch.empty((len(lens0), 4, 192), dtype=torch.bfloat16, device="cuda")
        t["vn"] = torch.empty_like(t["kn"])
        t["k_idx"] = _raw_to_tensor(idx.k_idx, "bf16", "cuda")
        t["z"] = _raw_to_tensor(idx.z, "bf16", "cuda")
        t["q_idx"] = _raw_to_tensor(idx.q_idx, "bf16", "cuda")
        t["w"] = torch.from_numpy(idx.w).cuda()
        t["summ"] = torch.zeros((len(lens0), case.max_blocks * 8, 256), dtype=torch.uint8,
                                device="cuda")
        mfa.mfa_sparse_summarize(t["k_idx"], t["z"], t["lens"], t["summ"], block_table=t["table"])
        t["sel"] = torch.empty((len(lens0), 4, 512), dtype=torch.int32, device="cuda")
        t["nsel"] = torch.empty((len(lens0), 4), dtype=torch.int32, device="cuda")
        t["dense"] = torch.empty((len(lens0), 64, 192), dtype=torch.bfloat16, device="cuda")
        t["sparse"] = torch.empty_like(t["dense"])
        return t

    def step(t):
        mfa.mfa_kv_append(t["kn"], t["vn"], t["k"], t["v"], t["table"], t["lens"],
                          v_layout="subblock8")
        mfa.mfa_sparse_summarize_new(t["k_idx"], t["z"], t["lens"], t["summ"], 1,
                                     block_table=t["table"])
        mfa.mfa_sparse_select(t["q_idx"], t["w"], t["summ"], t["lens"], t["sel"], t["nsel"],
                              block_table=t["table"])
        mfa.mfa_sparse_attention(t["q"], t["k"], t["v"], t["table"], t["lens"], t["sel"],
                                 t["nsel"], t["sparse"], case.scale)
        mfa.mfa_decode_attention_gqa(t["q"], t["k"], t["v"], t["table"], t["lens"], t["dense"],
                                     case.scale, v_layout="subblock8")

    def load(t, s):
        t["kn"].copy_(_raw_to_tensor(news[s][0], "bf16", "cuda"))
        t["vn"].copy_(_raw_to_tensor(news[s][1], "bf16", "cuda"))

    eager = state()
    ref_steps = []
    for s in range(STEPS):
        load(eager, s)
        step(eager)
        ref_steps.append((eager["dense"].clone(), eager["sparse"].clone(), eager["summ"].clone()))
    torch.cuda.synchronize()

    warm = state()                        # warm-up outside capture (workspace allocation)
    load(warm, 0)
    step(warm)
    torch.cuda.synchronize()
    g = state()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g)
    torch.cuda.synchronize()
    assert torch.equal(g["lens"].cpu(), torch.from_numpy(lens0.astype(np.int32)))
    for s in range(STEPS):
        load(g, s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        dense, sparse, summ = ref_steps[s]
        assert torch.equal(g["dense"].view(torch.int16), dense.view(torch.int16)), s
        assert torch.equal(g["sparse"].view(torch.int16), sparse.view(torch.int16)), s
        assert torch.equal(g["summ"], summ), s
        assert torch.equal(g["lens"].cpu(), torch.from_numpy((lens0 + s + 1).astype(np.int32)))
    assert torch.equal(g["k"].view(torch.int16), eager["k"].view(torch.int16))
    assert torch.equal(g["v"].view(torch.int16), eager["v"].view(torch.int16))

    k, v, lens = case.k_cache, case.v_cache, lens0
    for s in range(STEPS):
        k, v, lens = kv_append(k, v, lens, news[s][0], news[s][1], new_format="bf16",
                               kv_format="bf16", block_table=case.block_table)
    assert np.array_equal(g["v"].cpu().view(torch.int16).numpy().view(np.uint16), v_by_subblock(v))
    ref = decode_attention(case.q, k, v, lens, case.scale, **case.oracle_kwargs())
    assert_parity(g["dense"], ref, "bf16", "captured loop, dense call")
    assert_parity(g["sparse"], ref, "bf16", "captured loop, sparse call")
