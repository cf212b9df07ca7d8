"""Decode calls captured in a HIP graph and replayed.

The library only enqueues kernels and reads the slot lengths and the block
table on the device at run time, so a captured call replays correctly after
the caller updates those buffers in place (the pages' decode loop replays a
captured step with fresh lengths: duck-llm chapter 7, graph replay and state
hygiene).  Every replay is checked bit for bit against an eager call on the
same inputs, with eager work and synchronisation between the replays.
"""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention
from workloads import make_decode_case

from gpu_helpers import assert_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("splits", [0, 3])
def test_graph_replay_matches_eager_with_fresh_lengths(splits, kv):
    # The cache is drawn for the longest lengths of the schedule (rows past
    # those are NaN); the replays run with shorter or equal lengths.
    schedule = [[900, 64, 0, 2500, 1], [901, 65, 1, 2501, 2], [1000, 128, 64, 2560, 63]]
    case = make_decode_case(301, batch=5, ctx_lens=schedule[-1], hq=64, hkv=1, d=256,
                            kv_format=kv, scale=1 / 16)
    t = to_device(case)
    lens = t["lens"]
    lens.copy_(torch.tensor(schedule[0], dtype=torch.int32))
    out_g = torch.full_like(t["out"], float("nan"))
    out_e = torch.full_like(t["out"], float("nan"))

    def call(out):
        mfa.mfa_decode_attention(t["q"], t["k"], t["v"], t["table"], lens, out, case.scale,
                                 k_scale=t["k_scale"], v_scale=t["v_scale"], num_splits=splits)

    call(out_e)                 # warm-up outside capture (allocates the workspace)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g)
    torch.cuda.synchronize()

    # Each replay sees the lengths written in place before it (a decode step
    # appends one token per active slot).
    for step, new_lens in enumerate(schedule):
        lens.copy_(torch.tensor(new_lens, dtype=torch.int32))
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        call(out_e)             # eager reference on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {step}"
        ref = decode_attention(case.q, case.k_cache, case.v_cache, np.array(new_lens), case.scale,
                               **case.oracle_kwargs())
        assert_parity(out_g, ref, kv, f"replay {step}")


def _replay_against_eager(call, outs_g, outs_e, before_each, steps):
    """Capture call(outs_g), then per step: update inputs, replay, run the
    eager call into outs_e, and require bit-identical outputs."""
    call(outs_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(outs_g)
    torch.cuda.synchronize()
    for step in range(steps):
        before_each(step)
        for o in outs_g:
            o.fill_(-1 if o.dtype == torch.int32 else float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o in outs_e:
            o.fill_(-1 if o.dtype == torch.int32 else float("nan"))
        call(outs_e)
        torch.cuda.synchronize()
        for a, b in zip(outs_g, outs_e):
            ia = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
            ib = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
            assert torch.equal(ia, ib), f"replay {step}"


def test_multi_token_graph_replay():
    # Two query tokens per sequence (token pairs); the lengths grow between
    # replays as a decode loop with one draft token would.
    schedule = [[900, 2, 64, 3000], [902, 4, 66, 3002], [1000, 130, 1, 3072]]
    case = make_decode_case(311, batch=4, ctx_lens=schedule[-1], hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case)
    from workloads import make_mtp_queries
    from gpu_helpers import _raw_to_tensor
    q = _raw_to_tensor(make_mtp_queries(312, batch=4, tq=2), "bf16", "cuda")
    lens = t["lens"]
    outs_g = [torch.empty((4, 2, 64, 256), dtype=torch.bfloat16, device="cuda")]
    outs_e = [torch.empty_like(outs_g[0])]

    def call(outs):
        mfa.mfa_decode_attention_mtp(q, t["k"], t["v"], t["table"], lens, outs[0], case.scale)

    _replay_against_eager(call, outs_g, outs_e,
                          lambda s: lens.copy_(torch.tensor(schedule[s], dtype=torch.int32)),
                          len(schedule))


def test_sparse_step_graph_replay():
    # Selection and attention captured together; the lengths move the
    # candidate set and the current block between replays.
    from oracle.codecs import bf16_bits_to_f64
    from oracle.sparse import block_summaries
    from workloads import make_sparse_indexer_inputs, v_by_subblock
    from gpu_helpers import _raw_to_tensor
    schedule = [[5000, 9, 4100], [5001, 17, 4107], [6000, 800, 4108]]
    case = make_decode_case(321, batch=3, ctx_lens=schedule[-1], hq=64, hkv=4, d=192,
                            kv_format="bf16")
    idx = make_sparse_indexer_inputs(322, batch=3, cap=case.max_blocks * 64)
    summ = np.zeros((3, case.max_blocks * 8, 256), np.uint8)
    for b, L in enumerate(case.ctx_lens):
        _, c = block_summaries(bf16_bits_to_f64(idx.k_idx[b]), bf16_bits_to_f64(idx.z[b]), int(L))
        summ[b, :len(c)] = c
    table = torch.from_numpy(case.block_table).cuda()
    lens = torch.tensor(schedule[0], dtype=torch.int32, device="cuda")
    q = _raw_to_tensor(case.q, "bf16", "cuda")
    k = _raw_to_tensor(case.k_cache, "bf16", "cuda")
    v = _raw_to_tensor(v_by_subblock(case.v_cache), "bf16", "cuda")
    q_idx = _raw_to_tensor(idx.q_idx, "bf16", "cuda")
    w = torch.from_numpy(idx.w).cuda()
    s = torch.from_numpy(summ).cuda()

    def bufs():
        return [torch.empty((3, 4, 512), dtype=torch.int32, device="cuda"),
                torch.empty((3, 4), dtype=torch.int32, device="cuda"),
                torch.empty((3, 64, 192), dtype=torch.bfloat16, device="cuda")]
    outs_g, outs_e = bufs(), bufs()

    def call(outs):
        sel, nsel, out = outs
        mfa.mfa_sparse_select(q_idx, w, s, lens, sel, nsel, block_table=table)
        mfa.mfa_sparse_attention(q, k, v, table, lens, sel, nsel, out, case.scale)

    def new_lengths(step):
        lens.copy_(torch.tensor(schedule[step], dtype=torch.int32))

    # (entries past num_selected are not written: both sides keep the fill)
    _replay_against_eager(call, outs_g, outs_e, new_lengths, len(schedule))
