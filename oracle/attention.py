"""Decode attention, written as its plain definition in fp64.  TEST INFRASTRUCTURE ONLY.

Follows:
* "Step-3 is Large yet Affordable", section 2 (Step-3 model card) and Table 1:
  64 query heads share one K head and one V head, both of width 256.
* "Step-5-Preview: Sparse GQA, Indexer und KV-Speicher", section "Die
  eigentliche Attention liest weiterhin originale K/V", attention equation:
  head h reads KV group g(h) = floor(h / (Hq/Hkv)); softmax of scaled dot
  products over the attended keys, then the probability-weighted sum of V.
  Backbone table of the same page: the 512-token window includes the current
  token.
* duck-llm chapter 7, section 7.6 (decode context kernel): the active length
  passed to decode attention counts the token appended in this step.
* Paged caches (vLLM-style block tables, Step-3 report section 8.1; "page
  tables" in the Step-5 cache section) and static contiguous caches (duck-llm
  section 7.2).

Storage layouts (the same ones the HIP library documents):
  paged       K: [num_blocks, Hkv, P, d]     V: [num_blocks, Hkv, d, P]
  contiguous  K: [B, cap, Hkv, d]            V: [B, Hkv, d, cap]
with P = tokens per block.  Logical position j of slot b lives in block
block_table[b, j // P] at row j % P.  V blocks are stored channel-major
(d before tokens); the oracle simply indexes them as such.

Nothing here is blocked, fused or reordered: per slot, gather the attended
keys in logical order, decode to fp64, S = scale * q K^T, stable softmax,
out = P V.
"""

import numpy as np

from .codecs import decode_storage


def _gather_slot(k_cache, v_cache, block_table, b, positions, paged):
    """Return raw K rows [n, Hkv, d] and raw V rows [n, Hkv, d] for the listed
    logical positions of slot b (a plain walk of the block table)."""
    if paged:
        page = k_cache.shape[2]
        blocks = np.asarray(block_table[b], dtype=np.int64)[positions // page]
        rows = positions % page
        k = k_cache[blocks, :, rows, :]                 # [n, Hkv, d]
        v = v_cache[blocks, :, :, rows]                 # [n, Hkv, d]
    else:
        k = k_cache[b, positions, :, :]                 # [n, Hkv, d]
        v = np.transpose(v_cache[b][:, :, positions], (2, 0, 1))  # [n, Hkv, d]
    return k, v


def decode_attention(q, k_cache, v_cache, ctx_lens, scale, *, q_format, kv_format,
                     block_table=None, window=0, k_scale=None, v_scale=None,
                     slots=None):
    """fp64 decode attention.

    q          raw [B, Hq, d]  (float32 for "f32", uint16 bf16 bits for "bf16")
    k_cache    raw K storage, layout above; v_cache likewise
    ctx_lens   [B] ints, number of keys of each slot, current token included
    scale      logit scale (1/sqrt(d) on both pages' models)
    kv_format  "f32" | "bf16" | "e4m3"; for "e4m3" k_scale/v_scale are the
               per-KV-head fp32 dequantisation scales, value = code * scale
    window     0 = dense; W > 0 = keys [max(0, L - W), L - 1]
    slots      optional list of slot indices to evaluate (others skipped)

    Returns float64 [len(slots), Hq, d].  A slot with L == 0 yields zeros.
    """
    q = np.asarray(q)
    batch, hq, d = q.shape
    paged = block_table is not None
    hkv = k_cache.shape[1] if paged else k_cache.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if slots is None:
        slots = range(batch)
    slots = list(slots)
    out = np.zeros((len(slots), hq, d), dtype=np.float64)
    for i, b in enumerate(slots):
        L = int(ctx_lens[b])
        if L <= 0:
            continue
        lo = 0 if window <= 0 else max(0, L - window)
        positions = np.arange(lo, L, dtype=np.int64)
        k_raw, v_raw = _gather_slot(k_cache, v_cache, block_table, b, positions, paged)
        K = decode_storage(k_raw, kv_format)            # [n, Hkv, d]
        V = decode_storage(v_raw, kv_format)
        if kv_format == "e4m3":
            K = K * np.asarray(k_scale, dtype=np.float64)[None, :, None]
            V = V * np.asarray(v_scale, dtype=np.float64)[None, :, None]
        Q = decode_storage(q[b], q_format)              # [Hq, d]
        for h in range(hq):
            g = h // group
            s = scale * (K[:, g, :] @ Q[h])             # [n]
            m = np.max(s)
            e = np.exp(s - m)
            p = e / np.sum(e)
            out[i, h, :] = p @ V[:, g, :]
    return out


def softmax_weights(q, k_cache, ctx_lens, scale, *, q_format, kv_format, block_table=None,
                    window=0, k_scale=None, slot=0, head=0):
    """The probability row P[j] of one (slot, head): exposed so tests can check
    that the softmax rows sum to one and that masking selects the right keys."""
    q = np.asarray(q)
    paged = block_table is not None
    hkv = k_cache.shape[1] if paged else k_cache.shape[2]
    group = q.shape[1] // hkv
    L = int(ctx_lens[slot])
    lo = 0 if window <= 0 else max(0, L - window)
    positions = np.arange(lo, L, dtype=np.int64)
    if paged:
        page = k_cache.shape[2]
        blocks = np.asarray(block_table[slot], dtype=np.int64)[positions // page]
        k_raw = k_cache[blocks, :, positions % page, :]
    else:
        k_raw = k_cache[slot, positions, :, :]
    K = decode_storage(k_raw, kv_format)
    if kv_format == "e4m3":
        K = K * np.asarray(k_scale, dtype=np.float64)[None, :, None]
    Q = decode_storage(q[slot], q_format)
    g = head // group
    s = scale * (K[:, g, :] @ Q[head])
    e = np.exp(s - np.max(s))
    return positions, e / np.sum(e)
