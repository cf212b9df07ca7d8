"""Host logic of the attention latency-model fit (the attention-FFN ratio
page: t_A = alpha_A * T + beta_A, and the horizon-average token load
B (mu_P + mu_D) of its geometric workload model).  Pinned against a closed
form (two points), exact lines, and a direct simulation of the page's slot
process."""

import numpy as np
import pytest

from decode_attention_mfa_amd.accounting import fit_latency_model, horizon_token_load


def test_exact_line_is_recovered():
    T = np.array([8 * 512, 64 * 4096, 16 * 8192, 256 * 1024, 128 * 2048], dtype=float)
    alpha, beta = 0.19e-9, 4.5e-6
    a, b, r2 = fit_latency_model(T, alpha * T + beta)
    assert a == pytest.approx(alpha, rel=1e-9) and b == pytest.approx(beta, rel=1e-9)
    assert r2 == pytest.approx(1.0)


def test_two_points_give_the_secant():
    T1, T2, t1, t2 = 1.0e5, 9.0e5, 30e-6, 180e-6
    a, b, _ = fit_latency_model([T1, T2], [t1, t2])
    assert a == pytest.approx((t2 - t1) / (T2 - T1))
    assert b == pytest.approx(t1 - (t2 - t1) / (T2 - T1) * T1)


def test_noise_lowers_r2_and_degenerate_loads_are_rejected():
    rng = np.random.default_rng(1)
    T = np.linspace(1e5, 1e6, 12)
    a, b, r2 = fit_latency_model(T, 2e-10 * T + 5e-6 + rng.normal(0, 5e-6, T.size))
    assert 0.5 < r2 < 1.0 and a == pytest.approx(2e-10, rel=0.2)
    with pytest.raises(ValueError):
        fit_latency_model([5.0, 5.0], [1.0, 2.0])


def test_horizon_load_matches_the_slot_process():
    # The page's process: each step a slot continues with probability 1 - p
    # (decode index + 1) or is replaced by a new request (index 0, a fresh
    # prefill length of mean mu_P).  The long-run mean of T_k = sum of the
    # slots' prefill + decode lengths is B (mu_P + (1 - p) / p).
    B, p, mu_p, steps = 32, 1 / 300, 200.0, 60000
    rng = np.random.default_rng(7)
    s = rng.integers(100, 301, size=B).astype(float)      # prefill ~ U{100..300}, mean 200
    i = np.zeros(B)
    total = 0.0
    burn = 3000
    for k in range(steps):
        if k >= burn:
            total += float(np.sum(s + i))
        keep = rng.random(B) < 1 - p
        i = np.where(keep, i + 1, 0)
        s = np.where(keep, s, rng.integers(100, 301, size=B))
    assert total / (steps - burn) == pytest.approx(horizon_token_load(B, mu_p, p), rel=0.05)
