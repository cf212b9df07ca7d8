"""Algorithmic work of one decode-attention call (bytes moved, FLOPs).

Per slot with n attended keys (n = L, or min(L, W) for a window):
    bytes = 2 * Hkv * d * b_kv * n            K and V of the attended keys
          + Hq * d * (b_q + b_out)            the query token and its output
          + 4 * pages_touched + 4             block-table entries and the length
    FLOPs = 4 * Hq * d * n                    2 for QK^T and 2 for PV per key and channel
plus 8 * Hkv bytes of FP8 scales per call.  Split partials, padded tail rows
and re-reads are not algorithmic and are not counted.

The same per-key model reproduces the Step-3 report's accounting (section 4.1,
Tables 2 and 3: per-token KV bytes and attention FLOPs summed over 61
layers; section 5.1: arithmetic intensity 128 with 8-bit KV; section 7:
512 bytes of KV per token per layer) and the Step-5-Preview page's cache
formula (section "Cache-Kapazitaet": 2 * 4 * 192 * 2 = 3072 bytes per token
per layer in bf16); see tests/golden/pages_accounting.json.
"""

import math

PAGE = 64
DTYPE_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}


def kv_bytes_per_token(hkv, d, kv_bytes):
    """K plus V bytes of one cached token in one layer."""
    return 2 * hkv * d * kv_bytes


def attention_flops_per_key(hq, d):
    """QK^T plus PV FLOPs of one query token against one key."""
    return 4 * hq * d


def attended_keys(L, window=0):
    return min(L, window) if window > 0 else L


def pages_touched(L, window=0):
    if L <= 0:
        return 0
    lo = max(0, L - window) if window > 0 else 0
    return (L - 1) // PAGE - lo // PAGE + 1


def decode_call_bytes(ctx_lens, *, hq, hkv, d, q_fmt, kv_fmt, out_fmt, window=0):
    kvb = DTYPE_BYTES[kv_fmt]
    total = 0
    for L in ctx_lens:
        L = int(L)
        n = attended_keys(L, window)
        total += kv_bytes_per_token(hkv, d, kvb) * n
        total += hq * d * (DTYPE_BYTES[q_fmt] + DTYPE_BYTES[out_fmt])
        total += 4 * pages_touched(L, window) + 4
    if kv_fmt == "e4m3":
        total += 8 * hkv
    return total


def decode_call_flops(ctx_lens, *, hq, d, window=0):
    return sum(attention_flops_per_key(hq, d) * attended_keys(int(L), window) for L in ctx_lens)


def per_token_model(layers, context, *, hq, hkv, d, kv_bytes):
    """(KV bytes, attention FLOPs) to decode one token at a given context,
    summed over layers -- the form of the Step-3 report's Tables 2 and 3."""
    return (layers * context * kv_bytes_per_token(hkv, d, kv_bytes),
            layers * context * attention_flops_per_key(hq, d))


def query_proj_work(batch, hidden=7168, rank=2048, heads=64, head_dim=256):
    """(bytes, FLOPs) of the low-rank query path in bf16 (weights + x + q)."""
    width = heads * head_dim
    nbytes = 2 * (hidden * rank + rank * width) + 2 * batch * (hidden + width)
    flops = 2 * batch * (hidden * rank + rank * width)
    return nbytes, flops


def ceil_div(a, b):
    return -(-a // b)


def gib(x):
    return x / 2 ** 30


def mib(x):
    return x / 2 ** 20


def step5_cache_payload(T, *, global_layers=23, local_layers=69, window=512, hkv=4, d=192,
                        summary_dim=256, block=8):
    """Step-5-Preview one-request cache payload (bytes): global K/V, local
    ring buffers, E4M3 block summaries."""
    per_tok = kv_bytes_per_token(hkv, d, 2)
    return (per_tok * global_layers * T, per_tok * local_layers * window,
            global_layers * math.ceil(T / block) * summary_dim)


# ---- attention latency model (attention-FFN ratio page) ----
# The page models one attention step's latency as linear in the batch's token
# load, t_A = alpha_A * T + beta_A (a roofline-based linear model, Section
# "three-regime analysis"), where T is the number of cached tokens the step's
# attention reads (sum of the slots' context lengths), and replaces the
# drifting expected load by its horizon average, which tends to
# T_bar = B * (mu_P + mu_D) with mu_D = (1 - p) / p for geometric decode
# lengths (Proposition 4.3 as the page restates it).

def horizon_token_load(batch, mu_p, p):
    """Large-N horizon-average token load B (mu_P + (1 - p) / p)."""
    return batch * (mu_p + (1.0 - p) / p)


def fit_latency_model(token_loads, times):
    """Least-squares line times = alpha * token_loads + beta.

    Returns (alpha, beta, r2): seconds per cached token, fixed seconds per
    step, and the coefficient of determination of the fit."""
    import numpy as np
    T = np.asarray(token_loads, dtype=np.float64)
    t = np.asarray(times, dtype=np.float64)
    if T.size < 2 or np.ptp(T) == 0:
        raise ValueError("need at least two distinct token loads")
    A = np.stack([T, np.ones_like(T)], axis=1)
    (alpha, beta), *_ = np.linalg.lstsq(A, t, rcond=None)
    resid = t - (alpha * T + beta)
    ss_tot = float(np.sum((t - t.mean()) ** 2))
    r2 = 1.0 - float(resid @ resid) / ss_tot if ss_tot > 0 else 1.0
    return float(alpha), float(beta), r2
