"""KV append with a device-owned length counter, as its plain definition.
TEST INFRASTRUCTURE ONLY.

Follows duck-llm chapter 7, section 7.6 (the decode context kernel): each
decode step writes the new token's K and V into the cache at the slot's
current length and advances that length, so the decode attention of the same
step counts the new token (the active length is the cached length plus one).
Section 7.5 keeps that counter on the device, so nothing is read back between
steps.  Position j of slot b lives in block ``block_table[b, j // P]`` at row
``j % P`` of a paged cache (P tokens per block), or at position j of the slot
in a static contiguous cache (section 7.2); layouts as in
:mod:`oracle.attention`.

FP8 caches store OCP E4M3FN codes with one scale per KV head (stored value =
code * scale).  The oracle encodes ``x / scale`` -- the quotient taken in
fp32, as the device takes it -- by brute force: the finite code whose value
is nearest, ties to the code with an even mantissa, magnitudes above the
largest finite value (448) saturated to it, NaN to the NaN code.  Nothing is
derived from the bit layout except through :func:`e4m3fn_codes_to_f64`.
"""

import numpy as np

from .codecs import e4m3fn_codes_to_f64

_MAGS = np.arange(0x7F, dtype=np.uint8)            # finite non-negative codes 0 .. 0x7E
_MAG_VALUES = e4m3fn_codes_to_f64(_MAGS)           # increasing


def e4m3fn_encode(values):
    """Nearest E4M3FN code (uint8) of each value (ties to even, saturating)."""
    x = np.asarray(values, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        sign = 0x80 if np.signbit(v) else 0
        if np.isnan(v):
            out[i] = sign | 0x7F
            continue
        a = min(abs(v), _MAG_VALUES[-1])
        dist = np.abs(_MAG_VALUES - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:                       # a tie between two neighbours
            best = best[(_MAGS[best] & 1) == 0]
        out[i] = sign | int(_MAGS[best[0]])
    return out.reshape(x.shape)


def _widen(raw, fmt):
    """The new values as fp32, exactly (bf16 bits or f32)."""
    if fmt == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    if fmt == "f32":
        return np.asarray(raw, dtype=np.float32)
    raise ValueError(fmt)


def kv_append(k_cache, v_cache, ctx_lens, k_new, v_new, *, new_format, kv_format,
              block_table=None, k_scale=None, v_scale=None, active=None, num_blocks=None):
    """Return (k_cache', v_cache', ctx_lens') after appending one token per slot.

    k_new, v_new  raw [B, Hkv, d] (uint16 bf16 bits or float32)
    kv_format     "bf16" (copy bits), "f32" (copy) or "e4m3" (encode x / scale)
    A slot is skipped when active[b] == 0, when its length is outside
    [0, capacity), or (paged) when the block id at its length is outside the
    pool.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    lens = np.array(ctx_lens, dtype=np.int64, copy=True)
    paged = block_table is not None
    if paged:
        page = k.shape[2]
        cap = block_table.shape[1] * page
        pool = k.shape[0] if num_blocks is None else num_blocks
    else:
        cap = k.shape[1]
    B, hkv, d = np.shape(k_new)
    for b in range(B):
        if active is not None and active[b] == 0:
            continue
        pos = int(lens[b])
        if pos < 0 or pos >= cap:
            continue
        for g in range(hkv):
            if kv_format == "e4m3":
                kq = np.float32(_widen(k_new[b, g], new_format)) / np.float32(k_scale[g])
                vq = np.float32(_widen(v_new[b, g], new_format)) / np.float32(v_scale[g])
                kval, vval = e4m3fn_encode(kq.astype(np.float32)), e4m3fn_encode(vq.astype(np.float32))
            else:
                kval, vval = k_new[b, g], v_new[b, g]
            if paged:
                blk = int(block_table[b, pos // page])
                if blk < 0 or blk >= pool:
                    break
                k[blk, g, pos % page, :] = kval
                v[blk, g, :, pos % page] = vval
            else:
                k[b, pos, g, :] = kval
                v[b, g, :, pos] = vval
        else:
            lens[b] = pos + 1
    return k, v, lens
