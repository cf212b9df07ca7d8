"""Multi-token decode queries (MTP drafts, speculative verification), written as
their plain definition in fp64.  TEST INFRASTRUCTURE ONLY.

Follows "Step-3 is Large yet Affordable", section 5.2 (discussion of
quantisation and MTP): with MTP several new tokens of a request attend the
same KV cache in one step, which multiplies the attention's arithmetic
intensity.  The page does not spell out the masking; the reading taken here is
the usual causal one.  The Tq new tokens of a sequence are already in its
cache as its last Tq keys (the length counts them, duck-llm chapter 7, section
7.6), and token t attends keys [0, L - (Tq - 1 - t)): itself and everything
before it.  A token left with no key gets zeros, as an empty slot does.

Each token is therefore an ordinary decode query over a shorter prefix of the
same cache, which is exactly how this oracle evaluates it (one call of
:func:`oracle.attention.decode_attention` per token index, with the shortened
lengths).
"""

import numpy as np

from .attention import decode_attention


def mtp_lengths(ctx_lens, tq):
    """Keys attended by token t of each sequence: [B, Tq] = L - (Tq - 1 - t),
    floored at 0."""
    L = np.asarray(ctx_lens, dtype=np.int64)[:, None]
    t = np.arange(tq, dtype=np.int64)[None, :]
    return np.maximum(L - (tq - 1 - t), 0)


def decode_attention_mtp(q, k_cache, v_cache, ctx_lens, scale, *, q_format, kv_format,
                         block_table=None, k_scale=None, v_scale=None, slots=None):
    """fp64 multi-token decode attention.

    q         raw [B, Tq, Hq, d]; the other arguments as decode_attention
              (dense attention: no window)
    ctx_lens  [B] keys per sequence, all Tq new tokens included
    Returns float64 [len(slots), Tq, Hq, d].
    """
    q = np.asarray(q)
    batch, tq, hq, d = q.shape
    slots = list(range(batch) if slots is None else slots)
    lens = mtp_lengths(ctx_lens, tq)
    out = np.zeros((len(slots), tq, hq, d), dtype=np.float64)
    for t in range(tq):
        out[:, t] = decode_attention(q[:, t], k_cache, v_cache, lens[:, t], scale,
                                     q_format=q_format, kv_format=kv_format,
                                     block_table=block_table, k_scale=k_scale,
                                     v_scale=v_scale, slots=slots)
    return out
