"""Step-5 sparse global attention for one decode token per request, written as
its definition in fp64.  TEST INFRASTRUCTURE ONLY.

Follows "Step-5-Preview: Sparse GQA, Indexer und KV-Speicher":
* section "Acht Tokens ergeben einen Such-Key - koordinatenweise": a complete
  block r of 8 tokens gets the summary c[r, d] = sum_j a[j, d] kI[j, d] with
  a[:, d] the softmax of the compression logits z[:, d] over the block's 8
  tokens, per coordinate d; the result is stored as E4M3 after rounding to
  bf16.
* section "Auswahl per gewichtetem ReLU-Score": for query position t,
  provider group g and block r, s = sum_h w[g, h] ReLU(Q8(qI[g, h]) . Q8(c[r]))
  with Q8 the E4M3 rounding (then widened exactly); only blocks
  r < floor(t / 8) compete for the 512 places, equal scores go to the lower
  block id, and the block holding t is added with its positions up to t.
* section "Die eigentliche Attention liest weiterhin originale K/V": head h
  (group g(h) = floor(h / 16)) takes the ordinary scaled-dot-product softmax
  over the selected original tokens J[t, g] of its group.

Readings (the page leaves them open): the decode token sits at t = L - 1 with
L the request's length counting it; E4M3 rounding is to nearest, ties to even,
saturating at +-448 (as the library's FP8 cache writes); the bf16 rounding of
a summary is to nearest even from its exact value.
"""

import numpy as np

from .attention import decode_attention
from .codecs import bf16_bits_to_f64, e4m3fn_codes_to_f64
from .kv_append import e4m3fn_encode

BLOCK = 8        # tokens per historical block
BUDGET = 512     # historical blocks selected per (request, group)


def bf16_round(x):
    """Nearest bf16 value (ties to even) of float64 values that are finite
    and inside the bf16 range; returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0)                  # 8 significant bits, numpy rounds half to even
    return np.ldexp(q / 256.0, e)


def e4m3_round(x):
    """Q8: the nearest E4M3FN value of x, widened back exactly."""
    return e4m3fn_codes_to_f64(e4m3fn_encode(np.asarray(x, dtype=np.float64)))


def block_summaries(k_idx, z, length):
    """Summaries of the complete blocks of one request.

    k_idx, z  [cap, 256] float values of the proxy keys and compression logits
    length    tokens of the request (blocks r < length // 8 are complete)
    Returns (exact [nb, 256] float64, codes [nb, 256] uint8 E4M3 of the bf16-
    rounded summaries)."""
    nb = int(length) // BLOCK
    width = np.shape(k_idx)[-1]
    k = np.asarray(k_idx, dtype=np.float64)[:nb * BLOCK].reshape(nb, BLOCK, width)
    zz = np.asarray(z, dtype=np.float64)[:nb * BLOCK].reshape(nb, BLOCK, width)
    e = np.exp(zz - zz.max(axis=1, keepdims=True))
    a = e / e.sum(axis=1, keepdims=True)          # softmax over the block, per coordinate
    c = (a * k).sum(axis=1)
    return c, e4m3fn_encode(bf16_round(c))


def indexer_scores(q_idx, w, c_codes, t):
    """s[g, r] for the candidate blocks r < t // 8.

    q_idx    [4, 4, 256] float values (group, search head, coordinate)
    w        [4, 4] signed search-head weights (prescale included)
    c_codes  [>= t // 8, 256] E4M3 codes of the summaries"""
    R = int(t) // BLOCK
    q8 = e4m3_round(q_idx)                                   # [4, 4, 256]
    c8 = e4m3fn_codes_to_f64(np.asarray(c_codes)[:R])        # stored codes are Q8 already
    dots = np.einsum("ghd,rd->ghr", q8, c8)
    return np.einsum("gh,ghr->gr", np.asarray(w, dtype=np.float64), np.maximum(dots, 0.0))


def select_blocks(scores, budget=BUDGET):
    """Per group: the budget highest-scoring candidate ids (ties to the lower
    id), returned in ascending id order."""
    out = []
    for s in np.asarray(scores):
        order = sorted(range(len(s)), key=lambda r: (-s[r], r))
        out.append(np.array(sorted(order[:budget]), dtype=np.int64))
    return out


def attended_tokens(selected, t):
    """J[t, g]: the selected blocks' tokens and the current block up to t."""
    cur = (int(t) // BLOCK) * BLOCK
    hist = [np.arange(BLOCK * r, BLOCK * r + BLOCK) for r in selected]
    return np.concatenate(hist + [np.arange(cur, int(t) + 1)]).astype(np.int64)


def sparse_attention(q, k_cache, v_cache, block_table, b, t, selected, scale, *,
                     q_format="bf16", kv_format="bf16"):
    """Attention of request b's decode token (position t) over J[t, g] for
    every head.  q [Hq, d] raw; K paged as decode_attention, V^T stored per
    8-token sub-block, [blocks, Hkv, P/8, d, 8] (token j of a page in
    sub-block j // 8, column j % 8); selected is the per-group list of block
    ids.  Returns float64 [Hq, d]."""
    q = np.asarray(q)
    hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    page = k_cache.shape[2]
    for g in range(hkv):
        J = attended_tokens(selected[g], t)
        # Gather J into a contiguous one-request cache and run the dense oracle
        # on it (the order of J does not matter to a softmax).
        n = len(J)
        blocks = np.asarray(block_table[b], dtype=np.int64)[J // page]
        rows = J % page
        kc = k_cache[blocks, g, rows, :][None, :, None, :]                 # [1, n, 1, d]
        vc = np.transpose(v_cache[blocks, g, rows // BLOCK, :, rows % BLOCK], (1, 0))[None, None]   # [1, 1, d, n]
        qg = q[group * g:group * (g + 1)][None]
        out[group * g:group * (g + 1)] = decode_attention(
            qg, kc, vc, np.array([n]), scale, q_format=q_format, kv_format=kv_format)[0]
    return out


def sparse_decode(q, q_idx, w, c_codes, k_cache, v_cache, block_table, ctx_lens, scale, *,
                  slots=None):
    """The whole step for a batch: scores, selection, attention.  Returns
    (outputs [len(slots), Hq, d], selections per slot and group)."""
    slots = list(range(len(ctx_lens)) if slots is None else slots)
    outs, sels = [], []
    for b in slots:
        t = int(ctx_lens[b]) - 1
        if t < 0:
            outs.append(np.zeros(np.asarray(q).shape[1:], dtype=np.float64))
            sels.append([np.zeros(0, np.int64)] * 4)
            continue
        s = indexer_scores(bf16_bits_to_f64(q_idx[b]), w[b], c_codes[b], t)
        sel = select_blocks(s)
        outs.append(sparse_attention(q[b], k_cache, v_cache, block_table, b, t, sel, scale))
        sels.append(sel)
    return np.stack(outs), sels
