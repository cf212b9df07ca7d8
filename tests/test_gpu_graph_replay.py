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


@pytest.mark.parametrize("splits", [0, 3])
def test_graph_replay_matches_eager_with_fresh_lengths(splits):
    # The cache is drawn for the longest lengths of the schedule (rows past
    # those are NaN); the replays run with shorter or equal lengths.
    schedule = [[900, 64, 0, 2500, 1], [901, 65, 1, 2501, 2], [1000, 128, 64, 2560, 63]]
    case = make_decode_case(301, batch=5, ctx_lens=schedule[-1], hq=64, hkv=1, d=256,
                            scale=1 / 16)
    t = to_device(case)
    lens = t["lens"]
    lens.copy_(torch.tensor(schedule[0], dtype=torch.int32))
    out_g = torch.full_like(t["out"], float("nan"))
    out_e = torch.full_like(t["out"], float("nan"))

    def call(out):
        mfa.mfa_decode_attention(t["q"], t["k"], t["v"], t["table"], lens, out, case.scale,
                                 num_splits=splits)

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
        assert_parity(out_g, ref, "bf16", f"replay {step}")
