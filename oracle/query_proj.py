"""Low-rank MFA query path in fp64.  TEST INFRASTRUCTURE ONLY.

Follows "Step-3 is Large yet Affordable", section 2 (Step-3 model card) and
Table 1: the query is projected from the 7168-wide hidden state down to a
2048 rank, normalised, then projected up to 64 heads x 256.  The page says
only "normalised"; the reading used here (the workload's stated RMSNorm) is

    y = x W_down                       [B, rank]
    r = y / sqrt(mean(y^2) + eps) * g  (eps inside the root, gain g, no centring)
    q = reshape(r W_up, [B, heads, head_dim])   head h = columns h*hd .. h*hd+hd-1

Weights are row-major [in, out] so that y = x W.  Nothing is rounded.
"""

import numpy as np

from .codecs import decode_storage


def rms_norm(y, eps, gain=None):
    """Root-mean-square normalisation over the last axis (fp64)."""
    y = np.asarray(y, dtype=np.float64)
    r = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    if gain is not None:
        r = r * np.asarray(gain, dtype=np.float64)
    return r


def query_proj(x, w_down, w_up, *, fmt="bf16", eps=1e-6, gain=None, num_heads=64,
               head_dim=256):
    """x [B, hidden], w_down [hidden, rank], w_up [rank, num_heads*head_dim], all raw
    storage in `fmt` ("bf16" bits or "f32").  Returns float64 [B, num_heads, head_dim]."""
    X = decode_storage(x, fmt)
    Wd = decode_storage(w_down, fmt)
    Wu = decode_storage(w_up, fmt)
    if Wu.shape[1] != num_heads * head_dim:
        raise ValueError("w_up width must equal num_heads * head_dim")
    y = X @ Wd
    r = rms_norm(y, eps, gain)
    q = r @ Wu
    return q.reshape(X.shape[0], num_heads, head_dim)
