"""The device-side input generator, exercised on a CPU device: table and NaN
tail structure, and that the compact host copy of a few slots renumbers
blocks without changing any slot's data (the oracle gives the same answer on
the copy as on the full case)."""

import numpy as np
import torch

from oracle import decode_attention
from workloads.device_gen import make_device_case


def _case():
    return make_device_case(3, batch=4, ctx_lens=[1, 64, 130, 0], hq=8, hkv=2, d=32,
                            window=0, device="cpu")


def test_table_and_nan_tails():
    dc = _case()
    assert dc.block_table.shape == (4, 3)
    used = dc.block_table[dc.block_table >= 0]
    assert sorted(used.tolist()) == list(range(1 + 1 + 3))       # every pool block used once
    assert (dc.block_table[3] == -1).all()
    k = dc.k.float().numpy()
    v = dc.v.float().numpy()
    last = dc.block_table[2, 2]                                   # slot 2: 130 keys -> 2 rows
    assert np.isnan(k[last, :, 2:, :]).all() and np.isfinite(k[last, :, :2, :]).all()
    assert np.isnan(v[last, :, :, 2:]).all() and np.isfinite(v[last, :, :, :2]).all()
    full = dc.block_table[1, 0]                                   # slot 1: one whole block
    assert np.isfinite(k[full]).all()


def test_host_slots_keep_each_slots_data():
    dc = _case()
    whole = dc.host_slots([0, 1, 2, 3])
    part = dc.host_slots([2, 0])
    ref = decode_attention(whole.q, whole.k_cache, whole.v_cache, whole.ctx_lens, whole.scale,
                           **whole.oracle_kwargs())
    got = decode_attention(part.q, part.k_cache, part.v_cache, part.ctx_lens, part.scale,
                           **part.oracle_kwargs())
    np.testing.assert_array_equal(got, ref[[2, 0]])


def test_seeded():
    a, b = _case(), _case()
    assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16))
    assert np.array_equal(a.block_table, b.block_table)


def test_e4m3_scales_and_codes():
    dc = make_device_case(4, batch=3, ctx_lens=[70, 1, 128], hq=8, hkv=2, d=32,
                          kv_format="e4m3", device="cpu")
    assert dc.k.dtype == torch.float8_e4m3fn and dc.k_scale.shape == (2,)
    codes = dc.k.view(torch.uint8).numpy()
    last = dc.block_table[0, 1]                                   # slot 0: 70 keys -> 6 rows
    assert (codes[last, :, 6:, :] == 0x7F).all()
    valid = []                                                    # every valid row of the pool
    for b, L in enumerate(dc.ctx_lens):
        for j in range((int(L) + 63) // 64):
            rows = min(64, int(L) - 64 * j)
            valid.append(codes[dc.block_table[b, j], :, :rows, :].reshape(2, -1))
    valid = np.concatenate(valid, axis=1)
    assert ((valid & 0x7F) != 0x7F).all()                          # no NaN codes in valid rows
    assert ((valid & 0x7F) == 0x7E).any(axis=1).all()              # each head's absmax hits 448
    sub = dc.host_slots([2, 0])
    assert sub.kv_format == "e4m3" and sub.k_cache.dtype == np.uint8
    np.testing.assert_array_equal(sub.k_scale, dc.k_scale.numpy())
