"""Pins of the KV-append oracle (oracle/kv_append.py) against things other than
itself: the E4M3FN decoder round trip over every code, exact ties, saturation,
torch's own float8_e4m3fn cast on random values, and the attention oracle
reading back the appended token (duck-llm chapter 7, section 7.6: the length
the decode attention sees counts the token just written)."""

import numpy as np
import pytest
import torch

from oracle import decode_attention, decode_storage, e4m3fn_codes_to_f64, e4m3fn_encode, kv_append
from workloads import bf16_round_bits, make_decode_case


def bits(a):
    """Raw storage as integers, so that NaN rows compare equal to themselves."""
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    got = e4m3fn_encode(e4m3fn_codes_to_f64(codes))
    assert np.array_equal(got, codes)          # -0.0 (0x80) included


def test_nan_and_signed_zero():
    assert e4m3fn_encode(np.array([np.nan]))[0] == 0x7F
    assert e4m3fn_encode(np.array([-np.nan]))[0] == 0xFF
    assert e4m3fn_encode(np.array([-0.0]))[0] == 0x80
    assert e4m3fn_encode(np.array([-1e-30]))[0] == 0x80     # rounds to negative zero


def test_ties_go_to_the_even_code():
    mags = np.arange(0x7F, dtype=np.uint8)
    vals = e4m3fn_codes_to_f64(mags)
    mid = (vals[:-1] + vals[1:]) / 2
    lo, hi = mags[:-1], mags[1:]
    assert np.array_equal(e4m3fn_encode(mid), np.where((lo & 1) == 0, lo, hi))
    # just off the midpoint, the nearer code wins
    assert np.array_equal(e4m3fn_encode(np.nextafter(mid, 0)), lo)
    assert np.array_equal(e4m3fn_encode(np.nextafter(mid, np.inf)), hi)


def test_saturation_at_448():
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e4, np.inf, -500.0, -np.inf])
    assert list(e4m3fn_encode(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(3000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3fn_encode(x.astype(np.float64)), ref)


LENS = np.array([0, 1, 63, 64, 65, 127, 200], dtype=np.int64)


def _append_case(kv_format, seed=11, paged=True):
    # The tables hold a block for position L (room for L + 1 keys).
    case = make_decode_case(seed, batch=len(LENS), ctx_lens=LENS + 1, hq=8, hkv=2, d=16,
                            kv_format=kv_format, scale=0.25, paged=paged)
    rng = np.random.default_rng(seed + 1)
    new_fmt = "f32" if kv_format == "f32" else "bf16"

    def draw():
        x = rng.standard_normal((len(LENS), 2, 16)).astype(np.float32)
        return x if new_fmt == "f32" else bf16_round_bits(x)
    return case, draw(), draw(), new_fmt


def _run(case, k_new, v_new, new_fmt, kv_format, lens=LENS, **kw):
    return kv_append(case.k_cache, case.v_cache, lens, k_new, v_new, new_format=new_fmt,
                     kv_format=kv_format, block_table=kw.pop("table", case.block_table),
                     k_scale=case.k_scale, v_scale=case.v_scale, **kw)


@pytest.mark.parametrize("kv_format", ["bf16", "f32", "e4m3"])
def test_only_the_appended_rows_change(kv_format):
    case, k_new, v_new, new_fmt = _append_case(kv_format)
    k2, v2, lens2 = _run(case, k_new, v_new, new_fmt, kv_format)
    assert np.array_equal(lens2, LENS + 1)
    k_ref, v_ref = bits(case.k_cache).copy(), bits(case.v_cache).copy()
    for b, pos in enumerate(LENS):
        blk, row = case.block_table[b, pos // 64], pos % 64
        k_ref[blk, :, row, :] = bits(k2)[blk, :, row, :]
        v_ref[blk, :, :, row] = bits(v2)[blk, :, :, row]
    assert np.array_equal(bits(k2), k_ref) and np.array_equal(bits(v2), v_ref)


@pytest.mark.parametrize("kv_format", ["bf16", "f32", "e4m3"])
def test_appended_token_is_read_back_by_attention(kv_format):
    case, k_new, v_new, new_fmt = _append_case(kv_format)
    k2, v2, lens2 = _run(case, k_new, v_new, new_fmt, kv_format)
    # With q = 0 attention is the mean of V over the attended keys, so the
    # new token's V is (L+1) * out(after) - L * out(before): the attention
    # over the advanced length sees exactly the appended token.
    q = np.zeros((len(LENS), 8, 16), np.float32)
    kw = dict(q_format="f32", kv_format=kv_format, block_table=case.block_table,
              k_scale=case.k_scale, v_scale=case.v_scale)
    before = decode_attention(q, k2, v2, LENS, 1.0, **kw)
    after = decode_attention(q, k2, v2, lens2, 1.0, **kw)
    for b, pos in enumerate(LENS):
        blk, row = case.block_table[b, pos // 64], pos % 64
        for g in range(2):
            v = decode_storage(v2[blk, g, :, row], kv_format)
            v = v * (case.v_scale[g] if kv_format == "e4m3" else 1.0)
            got = (pos + 1) * after[b, 4 * g:4 * g + 4] - pos * before[b, 4 * g:4 * g + 4]
            assert np.allclose(got, v[None, :], rtol=0, atol=1e-10)
            assert np.array_equal(bits(v2)[blk, g, :, row], bits(_encoded(v_new, b, g, kv_format, case)))


def _encoded(v_new, b, g, kv_format, case):
    """What the cache must hold for the new V of (b, g): the bits for bf16 /
    f32, the nearest code of the fp32 quotient for FP8."""
    if kv_format != "e4m3":
        return v_new[b, g]
    x = (v_new[b, g].astype(np.uint32) << 16).view(np.float32)
    return e4m3fn_encode((x / np.float32(case.v_scale[g])).astype(np.float64))


def test_bf16_copies_bits_and_fp8_stores_the_nearest_code():
    case, k_new, v_new, _ = _append_case("bf16")
    k2, v2, _ = _run(case, k_new, v_new, "bf16", "bf16")
    for b, pos in enumerate(LENS):
        blk, row = case.block_table[b, pos // 64], pos % 64
        assert np.array_equal(k2[blk, :, row, :], k_new[b])
        assert np.array_equal(v2[blk, :, :, row], v_new[b])
    case8, k_new, v_new, _ = _append_case("e4m3")
    k2, _, _ = _run(case8, k_new, v_new, "bf16", "e4m3")
    grid = e4m3fn_codes_to_f64(np.arange(0x7F, dtype=np.uint8))
    for b, pos in enumerate(LENS):
        blk, row = case8.block_table[b, pos // 64], pos % 64
        for g in range(2):
            x = (k_new[b, g].astype(np.uint32) << 16).view(np.float32)
            quot = (x / np.float32(case8.k_scale[g])).astype(np.float64)
            got = e4m3fn_codes_to_f64(k2[blk, g, row, :])
            # no finite code lies nearer to the fp32 quotient than the stored one
            nearest = np.min(np.abs(grid[None, :] - np.abs(quot)[:, None]), axis=1)
            assert np.all(np.abs(np.abs(got) - np.abs(quot)) <= nearest)
            assert np.all((np.sign(got) == np.sign(quot)) | (got == 0))


def test_skipped_slots_keep_cache_and_length():
    case, k_new, v_new, _ = _append_case("bf16")
    table = case.block_table.copy()
    lens = LENS.copy()
    lens[1] = -1                            # negative length
    lens[2] = table.shape[1] * 64           # at capacity
    table[4, lens[4] // 64] = -1            # no block for the position
    active = np.ones(len(lens), np.int32)
    active[5] = 0                           # inactive slot
    k2, v2, out = _run(case, k_new, v_new, "bf16", "bf16", lens=lens, table=table, active=active)
    assert list(out) == [lens[0] + 1, -1, lens[2], lens[3] + 1, lens[4], lens[5], lens[6] + 1]
    k_ref, v_ref = bits(case.k_cache).copy(), bits(case.v_cache).copy()
    for b in (0, 3, 6):
        blk, row = table[b, lens[b] // 64], lens[b] % 64
        k_ref[blk, :, row, :] = k_new[b]
        v_ref[blk, :, :, row] = v_new[b]
    assert np.array_equal(bits(k2), k_ref) and np.array_equal(bits(v2), v_ref)


def test_contiguous_cache_positions():
    case, k_new, v_new, _ = _append_case("f32", paged=False)
    k2, v2, lens2 = _run(case, k_new, v_new, "f32", "f32", table=None)
    for b, pos in enumerate(LENS):
        assert np.array_equal(k2[b, pos, :, :], k_new[b])
        assert np.array_equal(v2[b, :, :, pos], v_new[b])
    assert np.array_equal(lens2, LENS + 1)
