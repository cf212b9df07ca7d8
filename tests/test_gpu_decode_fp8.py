"""GPU parity of MFA decode attention over an FP8 E4M3 cache (per-KV-head fp32
scales; single-token slots multiply K on the E4M3 matrix unit against a split
query, token pairs widen K to bf16) against the fp64 oracle.

Covers ragged lengths with NaN tail codes, every split count, fp32 output, the
contiguous cache, the windowed path, the full-size 256 x 4096 batch on
every slot (alone and fed by the query path), block permutations bit for bit, and a bit-exact check of the conversion of every finite code:
with a one-hot attention pattern the output is exactly the decoded V row."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention
from workloads import bf16_round_bits, make_decode_case
from workloads.device_gen import make_device_case

from gpu_helpers import assert_parity, run_decode, to_device

pytestmark = pytest.mark.gpu

RAGGED = [1, 63, 64, 65, 130, 1000, 0, 4096, 4033]


def oracle(case, slots=None):
    return decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                            slots=slots, **case.oracle_kwargs())


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_fp8_paged_ragged(splits):
    case = make_decode_case(90, batch=len(RAGGED), ctx_lens=RAGGED, hq=64, hkv=1, d=256,
                            kv_format="e4m3", scale=1 / 16)
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits)
    assert_parity(got, oracle(case), "e4m3", f"fp8 splits={splits}")


def test_fp8_fp32_output_and_contiguous_cache():
    case = make_decode_case(91, batch=4, ctx_lens=[5, 640, 0, 1111], hq=64, hkv=1, d=256,
                            kv_format="e4m3", paged=False, scale=1 / 16)
    t = to_device(case, out_format="f32")
    got = run_decode(case, t)
    assert got.dtype == torch.float32
    assert_parity(got, oracle(case), "e4m3", "fp8 contiguous, fp32 out")


@pytest.mark.parametrize("window", [1, 300])
def test_fp8_window(window):
    case = make_decode_case(92, batch=5, ctx_lens=[1, 64, 299, 1500, 4000], hq=64, hkv=1,
                            d=256, kv_format="e4m3", window=window, scale=1 / 16)
    t = to_device(case)
    for splits in (0, 3):
        got = run_decode(case, t, num_splits=splits)
        assert_parity(got, oracle(case), "e4m3", f"fp8 window={window} splits={splits}")


def test_fp8_query_dynamic_range():
    """Single-token slots over an E4M3 cache form S^T on the 8-bit matrix unit
    with each head's query scaled by a power of two and split into two E4M3
    terms.  Queries whose elements span 2^-20 .. 1 of one another (below
    ~2^-10 of a head's largest element the low term loses bits), heads
    scaled from 2^-12 to 2^3, a head of zeros and a head with a single
    non-zero element still meet the bar on every slot."""
    case = make_decode_case(95, batch=3, ctx_lens=[700, 64, 2049], hq=64, hkv=1, d=256,
                            kv_format="e4m3", scale=1 / 16)
    rng = np.random.default_rng(95)
    q = (case.q.astype(np.uint32) << 16).view(np.float32).reshape(case.batch, 64, 256).copy()
    q *= np.exp2(rng.integers(-20, 1, size=q.shape)).astype(np.float32)
    q[:, 20:36, :] *= np.exp2(np.arange(-12, 4)).astype(np.float32)[None, :, None]
    q[:, 5, :] = 0.0
    q[:, 9, :] = 0.0
    q[:, 9, 17] = 3.0
    case.q = bf16_round_bits(q)
    for splits in (0, 3):
        got = run_decode(case, to_device(case), num_splits=splits)
        assert_parity(got, oracle(case), "e4m3", f"fp8 query range splits={splits}", per_slot=True)


@pytest.mark.parametrize("jstar,splits", [(0, 1), (77, 0), (1000, 3), (1999, 4)])
def test_every_finite_code_decodes_exactly(jstar, splits):
    """q = 1, K code 448 on key j* and 0 elsewhere: the logit gap of
    256 * 448 / 16 = 7168 underflows every other weight to exactly 0, so with
    unit scales the output row equals the decoded V row, which holds every
    finite code."""
    L = 2000
    case = make_decode_case(93, batch=1, ctx_lens=[L], hq=64, hkv=1, d=256,
                            kv_format="e4m3", scale=1 / 16)
    case.q[:] = 0x3F80                                   # bf16 1.0
    case.k_scale[:] = 1.0
    case.v_scale[:] = 1.0
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                    # NaN codes -> 0
    blk, row = case.block_table[0, jstar // 64], jstar % 64
    valid_rows = np.arange(64)
    for i in range((L + 63) // 64):
        b = case.block_table[0, i]
        rows = valid_rows[valid_rows < L - 64 * i]
        case.k_cache[b, 0, rows, :] = 0
    case.k_cache[blk, 0, row, :] = 0x7E                  # 448
    case.v_cache[blk, 0, :, row] = codes                 # channel c holds code c
    t = to_device(case)
    got = run_decode(case, t, num_splits=splits).float().cpu().numpy()
    ref = oracle(case)
    np.testing.assert_array_equal(got, ref.astype(np.float32))


def _every_slot_oracle(dc, q_raw=None, q_format="bf16", chunk=64):
    """The oracle over every slot of a device case, copied back a chunk of
    slots at a time; q_raw replaces the case's query (format q_format)."""
    refs = []
    for s0 in range(0, dc.batch, chunk):
        slots = list(range(s0, min(dc.batch, s0 + chunk)))
        sub = dc.host_slots(slots)
        kw = sub.oracle_kwargs()
        kw["q_format"] = q_format
        q = sub.q if q_raw is None else q_raw[slots]
        refs.append(decode_attention(q, sub.k_cache, sub.v_cache, sub.ctx_lens, sub.scale, **kw))
    return np.concatenate(refs)


def test_config4_full_size_every_slot():
    """256 slots x 4096 keys, E4M3 K/V with per-head scales (drawn on the
    device), one split per slot as the benchmark runs it; every slot."""
    dc = make_device_case(4, batch=256, ctx_lens=[4096] * 256, hq=64, hkv=1, d=256,
                          kv_format="e4m3", scale=1 / 16, name="c4")
    out = torch.full((256, 64, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_decode_attention(dc.q, dc.k, dc.v, dc.table, dc.lens, out, dc.scale,
                             k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    assert_parity(out, _every_slot_oracle(dc), "e4m3", "config 4", per_slot=True)


def test_fp8_ragged_balanced_every_slot():
    """The ragged continuous-batching shape (128 slots, prefill ~ U[1024,
    8192] plus a geometric decode index) over an E4M3 cache drawn on the
    device: the heuristic's balanced page cut (slots cut into pieces across
    workgroups, single-token slots on the E4M3 S^T product) meets the bar on
    every slot."""
    from workloads import ragged_lengths
    lens = ragged_lengths(128)(np.random.default_rng(33))
    dc = make_device_case(33, batch=128, ctx_lens=lens, hq=64, hkv=1, d=256,
                          kv_format="e4m3", scale=1 / 16, name="c3-fp8")
    out = torch.full((128, 64, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    mfa.mfa_decode_attention(dc.q, dc.k, dc.v, dc.table, dc.lens, out, dc.scale,
                             k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    assert_parity(out, _every_slot_oracle(dc), "e4m3", "ragged fp8", per_slot=True)


def test_config4_query_path_into_fp8_attention_every_slot():
    """Config 4 as one chain: the low-rank query path (x [256, 7168] ->
    W_qdown -> RMSNorm -> W_qup -> 64 x 256, bf16 weights) feeds FP8-cache
    attention on the device, against the oracle's query path feeding its
    attention with the exact fp64 query ("Step-3 is Large yet Affordable",
    section 2).  The library's query is bf16, so its rounding is inside the
    tolerance here, unlike the per-step tests."""
    from oracle import query_proj
    from workloads import config_query_inputs
    qi = config_query_inputs(4, batch=256)
    dev = "cuda"

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.empty((256, 64 * 256), dtype=torch.bfloat16, device=dev)
    mfa.mfa_query_proj(bf16(qi.x), bf16(qi.w_down.T), bf16(qi.w_up.T), q, num_heads=64,
                       eps=qi.eps)
    dc = make_device_case(4, batch=256, ctx_lens=[4096] * 256, hq=64, hkv=1, d=256,
                          kv_format="e4m3", scale=1 / 16, name="c4")
    out = torch.full((256, 64, 256), float("nan"), dtype=torch.bfloat16, device=dev)
    mfa.mfa_decode_attention(q.view(256, 64, 256), dc.k, dc.v, dc.table, dc.lens, out, dc.scale,
                             k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    q_ref = query_proj(qi.x, qi.w_down, qi.w_up, fmt="bf16", eps=qi.eps, num_heads=64,
                       head_dim=256)
    ref = _every_slot_oracle(dc, q_raw=q_ref, q_format="f64")
    assert_parity(out, ref, "e4m3", "config 4 chain", per_slot=True)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_fp8_block_permutation_is_bit_exact(splits):
    # The same logical cache in the pool's identity order and shuffled: the
    # block-table walk must give bit-identical outputs.
    kw = dict(batch=4, ctx_lens=[777, 64, 2049, 4096], hq=64, hkv=1, d=256,
              kv_format="e4m3", scale=1 / 16)
    a = make_decode_case(94, shuffle=False, **kw)
    b = make_decode_case(94, shuffle=True, **kw)
    assert not np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.k_scale, b.k_scale) and np.array_equal(a.v_scale, b.v_scale)
    ga = run_decode(a, to_device(a), num_splits=splits).clone()
    gb = run_decode(b, to_device(b), num_splits=splits).clone()
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))
