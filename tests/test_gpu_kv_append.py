"""GPU parity of the KV append (mfa_kv_append) against the oracle, bit for bit:
the whole cache after the call (only each slot's row at its length may
change), the advanced lengths, FP8 codes at ties / saturation / subnormals,
skipped slots, and a captured append + decode graph replayed step after step
(the length lives on the device: duck-llm chapter 7, sections 7.5 and 7.6)."""

import numpy as np
import pytest
import torch

import decode_attention_mfa_amd as mfa
from oracle import decode_attention, e4m3fn_codes_to_f64, kv_append
from workloads import bf16_round_bits, make_decode_case

from gpu_helpers import assert_parity, to_device, _raw_to_tensor

pytestmark = pytest.mark.gpu

LENS = np.array([0, 1, 63, 64, 65, 127, 200, 511], dtype=np.int64)


def _case(kv_format, *, hkv=2, d=16, paged=True, seed=21):
    # Room for position L of every slot (the cache holds L + 1 keys' blocks).
    return make_decode_case(seed, batch=len(LENS), ctx_lens=LENS + 1, hq=8 * hkv, hkv=hkv, d=d,
                            kv_format=kv_format, scale=0.25, paged=paged)


def _new_values(kv_format, shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    return x if kv_format == "f32" else bf16_round_bits(x)


def _bits(t):
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def _bits_np(a):
    a = np.asarray(a)
    return a.view(np.int32) if a.dtype == np.float32 else a


def _run_both(case, k_new, v_new, kv_format, *, lens=LENS, table=None, active=None):
    """Append on the GPU and in the oracle; return both (k, v, lens)."""
    t = to_device(case)
    table = case.block_table if table is None else table
    new_fmt = "f32" if kv_format == "f32" else "bf16"
    kn = _raw_to_tensor(k_new, new_fmt, "cuda")
    vn = _raw_to_tensor(v_new, new_fmt, "cuda")
    tab = torch.from_numpy(table).cuda() if table is not None else None
    dlens = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    act = torch.from_numpy(active).cuda() if active is not None else None
    mfa.mfa_kv_append(kn, vn, t["k"], t["v"], tab, dlens, k_scale=t["k_scale"],
                      v_scale=t["v_scale"], active=act)
    torch.cuda.synchronize()
    ref = kv_append(case.k_cache, case.v_cache, lens, k_new, v_new, new_format=new_fmt,
                    kv_format=kv_format, block_table=table, k_scale=case.k_scale,
                    v_scale=case.v_scale, active=active)
    return (t["k"], t["v"], dlens), ref


def _assert_same(got, ref):
    (gk, gv, gl), (rk, rv, rl) = got, ref
    assert np.array_equal(gl.cpu().numpy().astype(np.int64), rl)
    assert np.array_equal(_bits(gk), _bits_np(rk))
    assert np.array_equal(_bits(gv), _bits_np(rv))


@pytest.mark.parametrize("kv_format,paged", [("bf16", True), ("e4m3", True), ("f32", True),
                                             ("bf16", False), ("f32", False)])
def test_append_matches_oracle_bit_for_bit(kv_format, paged):
    case = _case(kv_format, paged=paged)
    shape = (len(LENS), 2, 16)
    k_new, v_new = _new_values(kv_format, shape, 1), _new_values(kv_format, shape, 2)
    got, ref = _run_both(case, k_new, v_new, kv_format)
    _assert_same(got, ref)


def test_mfa_shape_append():
    # One KV head of width 256 (the MFA layout), 64 slots.
    lens = np.random.default_rng(5).integers(0, 700, size=64)
    case = make_decode_case(22, batch=64, ctx_lens=lens + 1, hq=64, hkv=1, d=256,
                            kv_format="bf16", scale=1 / 16)
    k_new, v_new = _new_values("bf16", (64, 1, 256), 3), _new_values("bf16", (64, 1, 256), 4)
    got, ref = _run_both(case, k_new, v_new, "bf16", lens=lens)
    _assert_same(got, ref)


def test_fp8_ties_saturation_and_subnormals():
    case = _case("e4m3", hkv=1, d=256)
    case.k_scale = np.array([2.0 ** -6], np.float32)   # powers of two: x / scale is exact
    case.v_scale = np.array([2.0 ** -3], np.float32)
    mags = e4m3fn_codes_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2                   # every tie, 126 of them
    vals = np.concatenate([mids, -mids, mags[:4], [0.0, -0.0, 600.0, -8192.0]])
    vals = np.resize(vals, (len(LENS), 1, 256)).astype(np.float32)
    k_new = bf16_round_bits(vals * np.float32(2.0 ** -6))
    v_new = bf16_round_bits(vals * np.float32(2.0 ** -3))
    # the constructed values are exactly representable, so the quotients are the ties
    assert np.array_equal((k_new.astype(np.uint32) << 16).view(np.float32) / np.float32(2.0 ** -6), vals)
    got, ref = _run_both(case, k_new, v_new, "e4m3")
    _assert_same(got, ref)


def test_skipped_slots_are_left_alone():
    case = _case("bf16")
    table = case.block_table.copy()
    lens = LENS.copy()
    lens[1] = -1                                   # negative length
    lens[2] = table.shape[1] * 64                  # at capacity
    table[4, lens[4] // 64] = -1                   # no block for the position
    table[6, lens[6] // 64] = case.k_cache.shape[0] + 5   # id outside the pool
    active = np.ones(len(lens), np.int32)
    active[5] = 0
    shape = (len(LENS), 2, 16)
    got, ref = _run_both(case, _new_values("bf16", shape, 7), _new_values("bf16", shape, 8), "bf16",
                         lens=lens, table=table, active=active)
    _assert_same(got, ref)


def test_captured_append_and_decode_replay_step_by_step():
    # A decode loop: each step appends one token per slot, then attends over
    # the advanced lengths.  Captured once; the new tokens are refreshed in
    # place before each replay; lengths advance on the device.
    steps = 3
    lens0 = np.array([5, 64, 130, 0, 1000, 63], dtype=np.int64)
    case = make_decode_case(23, batch=len(lens0), ctx_lens=lens0 + steps, hq=64, hkv=1, d=256,
                            kv_format="bf16", scale=1 / 16)
    news = [(_new_values("bf16", (len(lens0), 1, 256), 30 + 2 * s),
             _new_values("bf16", (len(lens0), 1, 256), 31 + 2 * s)) for s in range(steps)]

    def setup():
        t = to_device(case)
        t["lens"] = torch.from_numpy(lens0.astype(np.int32)).cuda()
        t["kn"] = torch.empty((len(lens0), 1, 256), dtype=torch.bfloat16, device="cuda")
        t["vn"] = torch.empty_like(t["kn"])
        return t

    def step(t):
        mfa.mfa_kv_append(t["kn"], t["vn"], t["k"], t["v"], t["table"], t["lens"])
        mfa.mfa_decode_attention(t["q"], t["k"], t["v"], t["table"], t["lens"], t["out"],
                                 case.scale)

    def load(t, s):
        t["kn"].copy_(_raw_to_tensor(news[s][0], "bf16", "cuda"))
        t["vn"].copy_(_raw_to_tensor(news[s][1], "bf16", "cuda"))

    eager = setup()
    eager_out = []
    for s in range(steps):
        load(eager, s)
        step(eager)
        eager_out.append(eager["out"].clone())
    torch.cuda.synchronize()

    g = setup()
    load(g, 0)
    warm = setup()                    # warm-up outside capture (workspace allocation)
    load(warm, 0)
    step(warm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g)
    torch.cuda.synchronize()
    # capture does not execute: the state is still the initial one
    assert torch.equal(g["lens"].cpu(), torch.from_numpy(lens0.astype(np.int32)))
    for s in range(steps):
        load(g, s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g["out"].view(torch.int16), eager_out[s].view(torch.int16)), s
        assert torch.equal(g["lens"].cpu(), torch.from_numpy((lens0 + s + 1).astype(np.int32)))
    assert torch.equal(g["k"].view(torch.int16), eager["k"].view(torch.int16))
    assert torch.equal(g["v"].view(torch.int16), eager["v"].view(torch.int16))

    # the oracle agrees with the final step
    k, v, lens = case.k_cache, case.v_cache, lens0
    for s in range(steps):
        k, v, lens = kv_append(k, v, lens, news[s][0], news[s][1], new_format="bf16",
                               kv_format="bf16", block_table=case.block_table)
    ref = decode_attention(case.q, k, v, lens, case.scale, q_format="bf16", kv_format="bf16",
                           block_table=case.block_table)
    assert_parity(g["out"], ref, "bf16", "append + decode, last replay")
