"""Pins for the oracle's decode attention (CPU only).

The oracle is checked against things other than itself:
* brute force: pure-Python loops with their own block-table walk, own bf16 /
  E4M3 widening (struct / torch) and math.exp, on tiny paged inputs with a
  4-token page, shuffled blocks, NaN tail rows, MQA and GQA, windows;
* torch's CPU scaled_dot_product_attention in float64 (library special case);
* closed forms and invariants: L = 1 returns V_0, constant V rows return the
  constant, q = 0 returns the mean of the attended V, softmax rows sum to one,
  physical block permutation leaves the result bit-identical, paged equals
  contiguous, MQA equals 64 independent single-head attentions, GQA head h
  equals single-head attention on group floor(h / (Hq/Hkv)), window >= L equals
  dense, window W equals dense attention over the last W keys, the length
  counts the current token, FP8 scales enter as value = code * scale.
"""

import math
import struct

import numpy as np
import pytest
import torch

from oracle import decode_attention
from oracle.attention import softmax_weights
from workloads import make_decode_case, bf16_round_bits


# ----------------------------------------------------------------------------------------
# brute force

def _bf16_scalar(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


_E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .to(torch.float64).tolist()


def _scalar(raw, fmt):
    if fmt == "f32":
        return float(raw)
    if fmt == "bf16":
        return _bf16_scalar(raw)
    return _E4M3[int(raw)]


def brute_force(q, kc, vc, lens, scale, table, window, q_fmt, kv_fmt, k_scale=None,
                v_scale=None):
    """Triple loops over (head, key, channel); paged layout K[blk,g,r,c], V[blk,g,c,r]."""
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    page = kc.shape[2]
    per_group = Hq // Hkv
    groups = [list(range(g * per_group, (g + 1) * per_group)) for g in range(Hkv)]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        first = 0 if window == 0 else max(0, L - window)
        keys = list(range(first, L))
        for h in range(Hq):
            g = [gi for gi, members in enumerate(groups) if h in members][0]
            ks = 1.0 if k_scale is None else float(k_scale[g])
            vs = 1.0 if v_scale is None else float(v_scale[g])
            logits = []
            for j in keys:
                blk = int(table[b][j // page])
                r = j % page
                acc = 0.0
                for c in range(d):
                    acc += _scalar(q[b, h, c], q_fmt) * (_scalar(kc[blk, g, r, c], kv_fmt) * ks)
                logits.append(scale * acc)
            top = max(logits)
            w = [math.exp(x - top) for x in logits]
            tot = sum(w)
            for c in range(d):
                acc = 0.0
                for wj, j in zip(w, keys):
                    blk = int(table[b][j // page])
                    acc += wj * (_scalar(vc[blk, g, c, j % page], kv_fmt) * vs)
                out[b, h, c] = acc / tot
    return out


def _tiny_paged(seed, lens, hq, hkv, d, page, kv_fmt, q_fmt):
    """Hand-built tiny paged case with a `page`-token page (the generator only
    makes 64-token pages), shuffled blocks and NaN tail rows."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens)
    nb = [(int(L) + page - 1) // page for L in lens]
    total = sum(nb)
    perm = rng.permutation(total)
    width = max(max(nb), 1)
    table = np.full((len(lens), width), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nb):
        for i in range(n):
            table[b, i] = perm[k]
            k += 1
    kf = rng.standard_normal((total, hkv, page, d)).astype(np.float32)
    vf = rng.standard_normal((total, hkv, d, page)).astype(np.float32)
    qf = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    k_scale = v_scale = None
    if kv_fmt == "bf16":
        kc, vc = bf16_round_bits(kf), bf16_round_bits(vf)
    elif kv_fmt == "e4m3":
        k_scale = np.array([0.03 + 0.01 * g for g in range(hkv)], dtype=np.float32)
        v_scale = np.array([0.02 + 0.005 * g for g in range(hkv)], dtype=np.float32)
        kc = rng.integers(0, 256, size=kf.shape).astype(np.uint8)
        vc = rng.integers(0, 256, size=vf.shape).astype(np.uint8)
        kc[(kc & 0x7F) == 0x7F] = 0x11
        vc[(vc & 0x7F) == 0x7F] = 0x22
    else:
        kc, vc = kf, vf
    q = bf16_round_bits(qf) if q_fmt == "bf16" else qf
    nan = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}[kv_fmt]
    for b, L in enumerate(lens):
        if L % page:
            blk = table[b, (int(L) - 1) // page]
            kc[blk, :, L % page:, :] = nan
            vc[blk, :, :, L % page:] = nan
    return q, kc, vc, table, k_scale, v_scale


@pytest.mark.parametrize("hq,hkv,window,kv_fmt,q_fmt", [
    (8, 1, 0, "bf16", "bf16"),
    (8, 2, 0, "bf16", "bf16"),
    (8, 2, 5, "f32", "f32"),
    (6, 3, 7, "e4m3", "bf16"),
    (4, 1, 3, "e4m3", "f32"),
])
def test_oracle_matches_brute_force(hq, hkv, window, kv_fmt, q_fmt):
    lens = [9, 1, 14, 0]
    d, page = 5, 4
    q, kc, vc, table, ks, vs = _tiny_paged(11 + hq + window, lens, hq, hkv, d, page, kv_fmt, q_fmt)
    scale = 0.37
    ref = brute_force(q, kc, vc, lens, scale, table, window, q_fmt, kv_fmt, ks, vs)
    got = decode_attention(q, kc, vc, np.array(lens), scale, q_format=q_fmt,
                           kv_format=kv_fmt, block_table=table, window=window,
                           k_scale=ks, v_scale=vs)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------
# library special case: torch SDPA (float64, CPU)

def _logical_kv(case, b):
    """Logical K, V [L, Hkv, d] of slot b via a vectorised walk (test-side code)."""
    from oracle.codecs import decode_storage
    L = int(case.ctx_lens[b])
    j = np.arange(L)
    if case.paged:
        blk = case.block_table[b][j // case.page]
        K = case.k_cache[blk, :, j % case.page, :]
        V = case.v_cache[blk, :, :, j % case.page]
    else:
        K = case.k_cache[b, :L]
        V = np.transpose(case.v_cache[b, :, :, :L], (2, 0, 1))
    K = decode_storage(K, case.kv_format)
    V = decode_storage(V, case.kv_format)
    if case.kv_format == "e4m3":
        K = K * case.k_scale[None, :, None]
        V = V * case.v_scale[None, :, None]
    return K, V


@pytest.mark.parametrize("kw", [
    dict(batch=3, ctx_lens=[130, 64, 1], hq=64, hkv=1, d=256, kv_format="bf16"),
    dict(batch=2, ctx_lens=[200, 77], hq=64, hkv=4, d=192, kv_format="bf16"),
    dict(batch=2, ctx_lens=[100, 65], hq=64, hkv=1, d=256, kv_format="e4m3"),
    dict(batch=2, ctx_lens=[128, 77], hq=64, hkv=1, d=256, kv_format="f32", paged=False),
])
def test_oracle_matches_torch_sdpa(kw):
    case = make_decode_case(5, **kw)
    got = decode_attention(case.q, case.k_cache, case.v_cache, case.ctx_lens, case.scale,
                           **case.oracle_kwargs())
    from oracle.codecs import decode_storage
    Q = decode_storage(case.q, case.q_format)
    G = case.hq // case.hkv
    for b in range(case.batch):
        K, V = _logical_kv(case, b)
        Kt = torch.from_numpy(np.ascontiguousarray(np.transpose(K, (1, 0, 2)))) \
            .repeat_interleave(G, dim=0)[None]
        Vt = torch.from_numpy(np.ascontiguousarray(np.transpose(V, (1, 0, 2)))) \
            .repeat_interleave(G, dim=0)[None]
        Qt = torch.from_numpy(Q[b])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, scale=case.scale)
        np.testing.assert_allclose(got[b], ref[0, :, 0, :].numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------------------
# closed forms and invariants

def _run(case, *, q=None, ctx_lens=None, scale=None, **over):
    kw = case.oracle_kwargs()
    kw.update(over)
    return decode_attention(case.q if q is None else q, case.k_cache, case.v_cache,
                            case.ctx_lens if ctx_lens is None else ctx_lens,
                            case.scale if scale is None else scale, **kw)


def test_single_key_returns_v0():
    case = make_decode_case(1, batch=2, ctx_lens=[1, 1], hq=64, hkv=1, d=256)
    out = _run(case)
    for b in range(2):
        _, V = _logical_kv(case, b)
        assert np.array_equal(out[b], np.broadcast_to(V[0, 0], (64, 256)))


def test_constant_values_return_the_constant():
    case = make_decode_case(2, batch=2, ctx_lens=[150, 64], hq=64, hkv=2, d=192)
    # every cached V entry of group g holds the same per-channel vector
    const = bf16_round_bits(np.random.default_rng(0).standard_normal((2, 192)).astype(np.float32))
    case.v_cache[:] = const[None, :, :, None]
    out = _run(case)
    from oracle.codecs import bf16_bits_to_f64
    c = bf16_bits_to_f64(const)
    for b in range(2):
        for h in range(64):
            np.testing.assert_allclose(out[b, h], c[h // 32], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("window", [0, 50])
def test_zero_query_gives_mean_of_attended_values(window):
    case = make_decode_case(3, batch=2, ctx_lens=[130, 33], hq=64, hkv=1, d=256, window=window)
    case.q[:] = 0
    out = _run(case)
    for b in range(2):
        _, V = _logical_kv(case, b)
        L = int(case.ctx_lens[b])
        lo = 0 if window == 0 else max(0, L - window)
        np.testing.assert_allclose(out[b, 7], V[lo:, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
    # scale = 0 is the same closed form
    case2 = make_decode_case(3, batch=2, ctx_lens=[130, 33], hq=64, hkv=1, d=256, window=window)
    out0 = decode_attention(case2.q, case2.k_cache, case2.v_cache, case2.ctx_lens, 0.0,
                            **case2.oracle_kwargs())
    np.testing.assert_allclose(out0, out, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("window", [0, 100])
def test_softmax_rows_sum_to_one_over_the_window(window):
    case = make_decode_case(4, batch=1, ctx_lens=[300], hq=64, hkv=1, d=256, window=window)
    pos, p = softmax_weights(case.q, case.k_cache, case.ctx_lens, case.scale,
                             q_format="bf16", kv_format="bf16", block_table=case.block_table,
                             window=window, slot=0, head=5)
    assert abs(p.sum() - 1.0) < 1e-12
    assert np.all(p > 0)
    lo = 0 if window == 0 else 300 - window
    assert np.array_equal(pos, np.arange(lo, 300))


def test_block_permutation_is_bit_identical():
    a = make_decode_case(7, batch=3, ctx_lens=[200, 64, 129], hq=64, hkv=1, d=256, shuffle=False)
    b = make_decode_case(7, batch=3, ctx_lens=[200, 64, 129], hq=64, hkv=1, d=256, shuffle=True)
    assert not np.array_equal(a.block_table, b.block_table)
    oa, ob = _run(a), _run(b)
    assert np.array_equal(oa, ob)


def test_paged_equals_contiguous():
    case = make_decode_case(8, batch=2, ctx_lens=[150, 64], hq=64, hkv=2, d=192)
    cap = 192
    kc = np.full((2, cap, 2, 192), 0x7FC0, dtype=np.uint16)
    vc = np.full((2, 2, 192, cap), 0x7FC0, dtype=np.uint16)
    for b in range(2):
        L = int(case.ctx_lens[b])
        j = np.arange(L)
        blk = case.block_table[b][j // 64]
        kc[b, :L] = case.k_cache[blk, :, j % 64, :]
        vc[b, :, :, :L] = np.transpose(case.v_cache[blk, :, :, j % 64], (1, 2, 0))
    paged = _run(case)
    contig = decode_attention(case.q, kc, vc, case.ctx_lens, case.scale, q_format="bf16",
                              kv_format="bf16", block_table=None)
    assert np.array_equal(paged, contig)


def test_mqa_equals_independent_single_head_attentions():
    case = make_decode_case(9, batch=2, ctx_lens=[97, 300], hq=64, hkv=1, d=256)
    full = _run(case)
    for h in (0, 13, 63):
        single = decode_attention(case.q[:, h:h + 1], case.k_cache, case.v_cache,
                                  case.ctx_lens, case.scale, q_format="bf16", kv_format="bf16",
                                  block_table=case.block_table)
        assert np.array_equal(full[:, h], single[:, 0])


def test_gqa_head_reads_group_floor_h_over_16():
    case = make_decode_case(10, batch=2, ctx_lens=[97, 70], hq=64, hkv=4, d=192)
    full = _run(case)
    for h in (0, 15, 16, 31, 47, 48, 63):
        g = h // 16
        single = decode_attention(case.q[:, h:h + 1], case.k_cache[:, g:g + 1],
                                  case.v_cache[:, g:g + 1], case.ctx_lens, case.scale,
                                  q_format="bf16", kv_format="bf16", block_table=case.block_table)
        assert np.array_equal(full[:, h], single[:, 0])
        # a modulo map would read another group: make sure that differs
        g_mod = h % 4
        if g_mod != g:
            other = decode_attention(case.q[:, h:h + 1], case.k_cache[:, g_mod:g_mod + 1],
                                     case.v_cache[:, g_mod:g_mod + 1], case.ctx_lens, case.scale,
                                     q_format="bf16", kv_format="bf16",
                                     block_table=case.block_table)
            assert not np.allclose(full[:, h], other[:, 0])


def test_window_at_least_length_equals_dense():
    case = make_decode_case(11, batch=3, ctx_lens=[100, 512, 37], hq=64, hkv=4, d=192)
    dense = _run(case, window=0)
    assert np.array_equal(_run(case, window=512), dense)
    assert np.array_equal(_run(case, window=10 ** 6), dense)
    assert not np.allclose(_run(case, window=99)[0], dense[0])


def test_window_equals_dense_over_last_w_keys():
    W = 70
    case = make_decode_case(12, batch=2, ctx_lens=[300, 90], hq=64, hkv=1, d=256, window=W)
    win = _run(case)
    for b in range(2):
        L = int(case.ctx_lens[b])
        j = np.arange(L - W, L)
        blk = case.block_table[b][j // 64]
        kc = case.k_cache[blk, :, j % 64, :][None]                       # [1, W, 1, d]
        vc = np.transpose(case.v_cache[blk, :, :, j % 64], (1, 2, 0))[None]  # [1, 1, d, W]
        dense = decode_attention(case.q[b:b + 1], kc, vc, np.array([W]), case.scale,
                                 q_format="bf16", kv_format="bf16", block_table=None)
        np.testing.assert_allclose(win[b], dense[0], rtol=1e-13, atol=1e-15)


def test_length_counts_the_current_token():
    case = make_decode_case(13, batch=1, ctx_lens=[129], hq=64, hkv=1, d=256)
    full = _run(case)
    minus_one = _run(case, ctx_lens=np.array([128]))
    assert not np.allclose(full, minus_one)


def test_one_hot_logits_return_that_value_row():
    case = make_decode_case(14, batch=1, ctx_lens=[200], hq=64, hkv=1, d=256)
    jstar = 131
    case.q[:] = bf16_round_bits(np.zeros((1, 64, 256), np.float32))
    case.q[:, :, 0] = bf16_round_bits(np.array([1.0], np.float32))[0]
    blk = case.block_table[0, jstar // 64]
    case.k_cache[blk, 0, jstar % 64, 0] = bf16_round_bits(np.array([4096.0], np.float32))[0]
    out = _run(case)
    _, V = _logical_kv(case, 0)
    np.testing.assert_allclose(out[0], np.broadcast_to(V[jstar, 0], (64, 256)), rtol=0, atol=1e-12)


def test_fp8_scales_enter_as_code_times_scale():
    case = make_decode_case(15, batch=2, ctx_lens=[130, 64], hq=64, hkv=1, d=256,
                            kv_format="e4m3")
    base = _run(case)
    twice_v = _run(case, v_scale=case.v_scale * 2)
    np.testing.assert_allclose(twice_v, 2 * base, rtol=1e-13, atol=1e-15)
    k2 = _run(case, k_scale=case.k_scale * 2)
    s2 = _run(case, scale=case.scale * 2)
    np.testing.assert_allclose(k2, s2, rtol=1e-12, atol=1e-14)


def test_empty_slot_gives_zeros_and_tails_are_never_read():
    case = make_decode_case(16, batch=3, ctx_lens=[0, 65, 1], hq=64, hkv=1, d=256)
    out = _run(case)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out))


def test_f64_query_is_taken_exactly():
    # The "f64" query format hands exact values to the definition: for queries
    # that are float32 values it equals the "f32" format bit for bit, and a
    # query off the float32 grid changes the result (nothing is rounded).
    case = make_decode_case(41, batch=2, ctx_lens=[70, 3], hq=8, hkv=2, d=64, kv_format="bf16")
    rng = np.random.default_rng(42)
    q32 = rng.standard_normal((2, 8, 64)).astype(np.float32)
    kw = case.oracle_kwargs()
    kw.pop("q_format")
    a = decode_attention(q32, case.k_cache, case.v_cache, case.ctx_lens, 0.125, q_format="f32", **kw)
    b = decode_attention(q32.astype(np.float64), case.k_cache, case.v_cache, case.ctx_lens, 0.125,
                         q_format="f64", **kw)
    assert np.array_equal(a, b)
    q64 = q32.astype(np.float64) + 1e-12
    c = decode_attention(q64, case.k_cache, case.v_cache, case.ctx_lens, 0.125, q_format="f64", **kw)
    assert not np.array_equal(a, c)
