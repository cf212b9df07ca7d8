"""Pins for the oracle's low-rank query path (CPU only): brute-force loops on
tiny shapes, the RMSNorm mean-square closed form, the head-major reshape, the
gain, and scale invariance of the normalised path."""

import math
import struct

import numpy as np
import pytest

from oracle import query_proj, rms_norm
from workloads import bf16_round_bits, make_query_inputs


def _f(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(x, wd, wu, eps, heads, hd, gain=None):
    B, H = x.shape
    R = wd.shape[1]
    out = np.zeros((B, heads, hd))
    for b in range(B):
        y = []
        for r in range(R):
            acc = 0.0
            for i in range(H):
                acc += _f(x[b, i]) * _f(wd[i, r])
            y.append(acc)
        ms = sum(v * v for v in y) / R
        inv = 1.0 / math.sqrt(ms + eps)
        z = [y[r] * inv * (1.0 if gain is None else gain[r]) for r in range(R)]
        for h in range(heads):
            for c in range(hd):
                col = h * hd + c
                out[b, h, c] = sum(z[r] * _f(wu[r, col]) for r in range(R))
    return out


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_query_proj_matches_brute_force(eps):
    rng = np.random.default_rng(3)
    qi = make_query_inputs(rng, batch=3, hidden=7, rank=5, num_heads=2, head_dim=3, eps=eps)
    got = query_proj(qi.x, qi.w_down, qi.w_up, eps=eps, num_heads=2, head_dim=3)
    ref = _brute(qi.x, qi.w_down, qi.w_up, eps, 2, 3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    gain = np.array([0.5, 2.0, -1.0, 1.5, 3.0])
    got_g = query_proj(qi.x, qi.w_down, qi.w_up, eps=eps, num_heads=2, head_dim=3, gain=gain)
    ref_g = _brute(qi.x, qi.w_down, qi.w_up, eps, 2, 3, gain=gain)
    np.testing.assert_allclose(got_g, ref_g, rtol=1e-12, atol=1e-14)


def test_rmsnorm_mean_square_closed_form():
    rng = np.random.default_rng(4)
    for eps, scale in [(1e-6, 1.0), (1e-6, 1e-3), (1e-2, 0.1)]:
        y = rng.standard_normal((4, 2048)) * scale
        r = rms_norm(y, eps)
        ms = np.mean(y * y, axis=1)
        np.testing.assert_allclose(np.mean(r * r, axis=1), ms / (ms + eps), rtol=1e-12)
        # direction unchanged, no centring
        np.testing.assert_allclose(r / np.linalg.norm(r, axis=1, keepdims=True),
                                   y / np.linalg.norm(y, axis=1, keepdims=True), rtol=1e-12)


def test_head_major_reshape():
    rng = np.random.default_rng(5)
    qi = make_query_inputs(rng, batch=2, hidden=16, rank=8, num_heads=4, head_dim=6)
    wu = np.zeros_like(qi.w_up)
    col = 3 * 6 + 4                      # head 3, channel 4
    wu[:, col] = bf16_round_bits(np.ones(8, np.float32))
    q = query_proj(qi.x, qi.w_down, wu, num_heads=4, head_dim=6)
    nz = np.argwhere(q[0] != 0)
    assert nz.tolist() == [[3, 4]]


def test_normalised_path_is_scale_invariant():
    rng = np.random.default_rng(6)
    qi = make_query_inputs(rng, batch=2, hidden=32, rank=16, num_heads=2, head_dim=4)
    q1 = query_proj(qi.x, qi.w_down, qi.w_up, eps=0.0, num_heads=2, head_dim=4)
    x8 = bf16_round_bits(np.float32(8.0) * (qi.x.astype(np.uint32) << 16).view(np.float32))
    q8 = query_proj(x8, qi.w_down, qi.w_up, eps=0.0, num_heads=2, head_dim=4)
    np.testing.assert_allclose(q8, q1, rtol=1e-12, atol=1e-13)
