"""Seeded synthetic decode-attention inputs.

Recipe (one numpy Generator per case, ``default_rng(seed)``), fixed draw order:
context lengths -> q -> K -> V -> block permutation.  The query-path inputs
(x, W_qdown, W_qup) come from a second generator ``default_rng([seed, 1])`` so
they can be drawn without drawing the cache.
Values are N(0, 1) drawn in float32; bf16 storage is the round-to-nearest-even
of that float32; FP8 storage is OCP E4M3FN produced by torch's float8_e4m3fn
cast of x / scale with one fp32 scale per KV head, scale = absmax / 448 over
that head's valid cached entries.  K and V are drawn token-major, one 64-token
logical block at a time in (slot, block) order; the pool position of logical
block k is ``perm[k]`` with ``perm = rng.permutation(num_blocks)``.

Cache layouts (the library's):
  paged       K [num_blocks, Hkv, P, d]     V [num_blocks, Hkv, d, P]
  contiguous  K [B, cap, Hkv, d]            V [B, Hkv, d, cap]
Rows past a slot's length inside its last block ("tail rows") hold NaN
(bf16 0x7FC0, f32 NaN, E4M3 0x7F) when ``nan_tail`` is set, so any read of
them that is not masked poisons the result; otherwise they hold random data.
Unused block-table entries are -1.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PAGE = 64
BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0

CONFIG_NAMES = {
    1: "tiny MFA decode, fp32, B=2, L={128,77}, contiguous cache",
    2: "Step-3-shaped MFA decode, bf16, B=64, L=4096, paged 64-token blocks",
    3: "ragged continuous-batching MFA decode, bf16, B=128, L=U[1024,8192]+Geo(1/1024)",
    4: "MFA query path + FP8 E4M3 KV, B=256, L=4096",
    5: "GQA 64/4/192, B=32, L=32768, window 512 (local) and dense (global)",
}


def bf16_round_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even; NaN -> 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN
    return out


def _e4m3_codes(x, scale):
    import torch  # the cast is torch's float8_e4m3fn conversion (RNE, saturating)
    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class DecodeCase:
    """One decode-attention call's inputs, as raw storage arrays (host)."""
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    d: int
    q_format: str                 # "f32" | "bf16"
    kv_format: str                # "f32" | "bf16" | "e4m3"
    out_format: str               # "f32" | "bf16"
    q: np.ndarray                 # [B, Hq, d] float32 or uint16 bits
    k_cache: np.ndarray
    v_cache: np.ndarray
    ctx_lens: np.ndarray          # [B] int32
    block_table: Optional[np.ndarray]  # [B, M] int32 or None (contiguous)
    scale: float
    window: int = 0
    k_scale: Optional[np.ndarray] = None   # [Hkv] float32 (e4m3 only)
    v_scale: Optional[np.ndarray] = None
    page: int = PAGE
    meta: dict = field(default_factory=dict)

    @property
    def paged(self):
        return self.block_table is not None

    @property
    def max_blocks(self):
        if self.paged:
            return int(self.block_table.shape[1])
        return int(self.k_cache.shape[1]) // self.page

    @property
    def num_blocks(self):
        return int(self.k_cache.shape[0]) if self.paged else 0

    def oracle_kwargs(self):
        return dict(q_format=self.q_format, kv_format=self.kv_format,
                    block_table=self.block_table, window=self.window,
                    k_scale=self.k_scale, v_scale=self.v_scale)


def _storage(x, fmt):
    if fmt == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "bf16":
        return bf16_round_bits(x)
    raise ValueError(fmt)


def make_decode_case(seed, *, batch, ctx_lens, hq=64, hkv=1, d=256, kv_format="bf16",
                     q_format=None, out_format=None, paged=True, window=0, scale=None,
                     nan_tail=True, shuffle=True, table_width=None, draw_q=True,
                     rng=None, name="custom", chunk_blocks=1024):
    """Build a DecodeCase.  ``ctx_lens`` is a sequence of ints or a callable
    ``rng -> lengths`` (drawn first, from the case's generator)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = ctx_lens(rng) if callable(ctx_lens) else ctx_lens
    lens = np.asarray(lens, dtype=np.int64)
    if lens.shape != (batch,):
        raise ValueError("ctx_lens must have one entry per slot")
    q_format = q_format or ("f32" if kv_format == "f32" else "bf16")
    out_format = out_format or ("f32" if kv_format == "f32" else "bf16")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nblk_slot = (lens + PAGE - 1) // PAGE
    width = int(nblk_slot.max()) if batch else 0
    if table_width is not None:
        if table_width < width:
            raise ValueError("table_width below the longest context")
        width = int(table_width)
    width = max(width, 1)

    q = None
    if draw_q:
        q = _storage(rng.standard_normal((batch, hq, d), dtype=np.float32), q_format)

    store = "bf16" if kv_format == "bf16" else "f32"   # e4m3 is quantised below

    if paged:
        nblk = int(nblk_slot.sum())
        k_log = np.empty((nblk, hkv, PAGE, d), dtype=np.float32)
        v_log = np.empty((nblk, hkv, PAGE, d), dtype=np.float32)
        for s in range(0, nblk, chunk_blocks):
            e = min(nblk, s + chunk_blocks)
            k_log[s:e] = rng.standard_normal((e - s, hkv, PAGE, d), dtype=np.float32)
        for s in range(0, nblk, chunk_blocks):
            e = min(nblk, s + chunk_blocks)
            v_log[s:e] = rng.standard_normal((e - s, hkv, PAGE, d), dtype=np.float32)
        perm = rng.permutation(nblk) if shuffle else np.arange(nblk)
        table = np.full((batch, width), -1, dtype=np.int32)
        valid = np.ones((nblk, PAGE), dtype=bool)       # token validity per logical block
        k = 0
        for b in range(batch):
            for i in range(int(nblk_slot[b])):
                table[b, i] = perm[k]
                tail = int(lens[b]) - i * PAGE
                if tail < PAGE:
                    valid[k, tail:] = False
                k += 1
        k_scale = v_scale = None
        if kv_format == "e4m3":
            mask = valid[:, None, :, None]
            k_scale = np.array([np.abs(np.where(mask, k_log, 0)[:, g]).max() / E4M3_MAX
                                for g in range(hkv)], dtype=np.float32)
            v_scale = np.array([np.abs(np.where(mask, v_log, 0)[:, g]).max() / E4M3_MAX
                                for g in range(hkv)], dtype=np.float32)
            k_raw = np.empty(k_log.shape, dtype=np.uint8)
            v_raw = np.empty(v_log.shape, dtype=np.uint8)
            for g in range(hkv):
                k_raw[:, g] = _e4m3_codes(k_log[:, g], k_scale[g])
                v_raw[:, g] = _e4m3_codes(v_log[:, g], v_scale[g])
            nan_code = E4M3_NAN
        else:
            k_raw = np.empty(k_log.shape, dtype=np.float32 if store == "f32" else np.uint16)
            v_raw = np.empty(v_log.shape, dtype=k_raw.dtype)
            for s in range(0, nblk, chunk_blocks):
                e = min(nblk, s + chunk_blocks)
                k_raw[s:e] = _storage(k_log[s:e], store)
                v_raw[s:e] = _storage(v_log[s:e], store)
            nan_code = np.float32(np.nan) if store == "f32" else BF16_NAN
        del k_log, v_log
        if nan_tail:
            inv = ~valid
            kb, rows = np.nonzero(inv)
            k_raw[kb, :, rows, :] = nan_code
            v_raw[kb, :, rows, :] = nan_code
        # place logical blocks at their pool positions; V stored channel-major
        k_cache = np.empty_like(k_raw)
        k_cache[perm] = k_raw
        del k_raw
        v_cache = np.empty((nblk, hkv, d, PAGE), dtype=v_raw.dtype)
        for s in range(0, nblk, chunk_blocks):
            e = min(nblk, s + chunk_blocks)
            v_cache[perm[s:e]] = np.transpose(v_raw[s:e], (0, 1, 3, 2))
        del v_raw
        block_table = table
    else:
        cap = width * PAGE
        k_log = rng.standard_normal((batch, cap, hkv, d), dtype=np.float32)
        v_log = rng.standard_normal((batch, cap, hkv, d), dtype=np.float32)
        valid = np.arange(cap)[None, :] < lens[:, None]         # [B, cap]
        k_scale = v_scale = None
        if kv_format == "e4m3":
            mask = valid[:, :, None, None]
            k_scale = np.array([np.abs(np.where(mask, k_log, 0)[:, :, g]).max() / E4M3_MAX
                                for g in range(hkv)], dtype=np.float32)
            v_scale = np.array([np.abs(np.where(mask, v_log, 0)[:, :, g]).max() / E4M3_MAX
                                for g in range(hkv)], dtype=np.float32)
            k_raw = np.stack([_e4m3_codes(k_log[:, :, g], k_scale[g]) for g in range(hkv)], axis=2)
            v_raw = np.stack([_e4m3_codes(v_log[:, :, g], v_scale[g]) for g in range(hkv)], axis=2)
            nan_code = E4M3_NAN
        else:
            k_raw = _storage(k_log, store)
            v_raw = _storage(v_log, store)
            nan_code = np.float32(np.nan) if store == "f32" else BF16_NAN
        if nan_tail:
            bb, jj = np.nonzero(~valid)
            k_raw[bb, jj] = nan_code
            v_raw[bb, jj] = nan_code
        k_cache = np.ascontiguousarray(k_raw)
        v_cache = np.ascontiguousarray(np.transpose(v_raw, (0, 2, 3, 1)))   # [B, Hkv, d, cap]
        block_table = None

    return DecodeCase(name=name, seed=seed, batch=batch, hq=hq, hkv=hkv, d=d,
                      q_format=q_format, kv_format=kv_format, out_format=out_format,
                      q=q, k_cache=k_cache, v_cache=v_cache,
                      ctx_lens=lens.astype(np.int32), block_table=block_table,
                      scale=float(scale), window=int(window), k_scale=k_scale,
                      v_scale=v_scale)


def make_mtp_queries(seed, *, batch, tq, hq=64, d=256, q_format="bf16"):
    """Tq new query tokens per slot, [B, Tq, Hq, d], N(0, 1) in the query
    storage format (multi-token decode: MTP drafts or a speculative verify)."""
    rng = np.random.default_rng(seed)
    return _storage(rng.standard_normal((batch, tq, hq, d), dtype=np.float32), q_format)


@dataclass
class SparseIndexerInputs:
    """Step-5 indexer inputs of a batch (raw storage): search queries
    q_idx [B, 4, 4, 256] and proxy keys / compression logits k_idx, z
    [B, cap, 256] as bf16 bits, search-head weights w [B, 4, 4] float32."""
    q_idx: np.ndarray
    w: np.ndarray
    k_idx: np.ndarray
    z: np.ndarray


def v_by_subblock(v_cache, block=8):
    """A paged V^T cache [blocks, Hkv, d, P] relaid per sub-block of `block`
    tokens: [blocks, Hkv, P / block, d, block] (data movement only)."""
    nb, hkv, d, page = v_cache.shape
    return np.ascontiguousarray(
        v_cache.reshape(nb, hkv, d, page // block, block).transpose(0, 1, 3, 2, 4))


def make_sparse_indexer_inputs(seed, *, batch, cap, groups=4, heads=4, width=256):
    """N(0, 1) search queries, proxy keys and logits (bf16); weights
    N(0, 1) * 4^-1/2, the prescale the page says the weights carry."""
    rng = np.random.default_rng(seed)
    q_idx = bf16_round_bits(rng.standard_normal((batch, groups, heads, width), dtype=np.float32))
    w = (rng.standard_normal((batch, groups, heads), dtype=np.float32) * np.float32(0.5))
    k_idx = bf16_round_bits(rng.standard_normal((batch, cap, width), dtype=np.float32))
    z = bf16_round_bits(rng.standard_normal((batch, cap, width), dtype=np.float32))
    return SparseIndexerInputs(q_idx=q_idx, w=w, k_idx=k_idx, z=z)


def ragged_lengths(batch, *, p_lo=1024, p_hi=8192, geo_p=1.0 / 1024, cap=32768):
    """Continuous-batching context lengths: prefill length ~ Uniform{p_lo..p_hi}
    plus a decode index ~ Geometric(p) on {0, 1, ...} (numpy counts trials from 1,
    hence the -1), capped.  Workload model of "Theoretically Optimal
    Attention/FFN Ratios in Disaggregated LLM Serving" (probabilistic workload
    model: geometric decode lengths, prefill entering through its mean)."""
    def draw(rng):
        prefill = rng.integers(p_lo, p_hi + 1, size=batch)
        decode_idx = rng.geometric(geo_p, size=batch) - 1
        return np.minimum(prefill + decode_idx, cap)
    return draw


@dataclass
class QueryInputs:
    x: np.ndarray        # [B, hidden] bf16 bits
    w_down: np.ndarray   # [hidden, rank] bf16 bits
    w_up: np.ndarray     # [rank, heads*head_dim] bf16 bits
    eps: float = 1e-6
    num_heads: int = 64
    head_dim: int = 256


def make_query_inputs(rng, *, batch, hidden=7168, rank=2048, num_heads=64, head_dim=256,
                      eps=1e-6):
    """x ~ N(0,1); W ~ N(0, 1/fan_in); all rounded to bf16 (row-major [in, out])."""
    x = bf16_round_bits(rng.standard_normal((batch, hidden), dtype=np.float32))
    wd = rng.standard_normal((hidden, rank), dtype=np.float32)
    wd *= np.float32(1.0 / np.sqrt(hidden))
    wd = bf16_round_bits(wd)
    wu = rng.standard_normal((rank, num_heads * head_dim), dtype=np.float32)
    wu *= np.float32(1.0 / np.sqrt(rank))
    wu = bf16_round_bits(wu)
    return QueryInputs(x=x, w_down=wd, w_up=wu, eps=eps, num_heads=num_heads,
                       head_dim=head_dim)


def config_case(n, *, nan_tail=True, window=None, seed=None):
    """The five benchmark shapes as DecodeCases (seed = config number by default).
    Config 4 has no drawn q: its q comes from the query path
    (see :func:`config_query_inputs`).  Config 5 takes ``window`` = 512 (local
    layer) or 0 (dense global layer); both read the same cache."""
    seed = n if seed is None else seed
    if n == 1:
        return make_decode_case(seed, batch=2, ctx_lens=[128, 77], hq=64, hkv=1, d=256,
                                kv_format="f32", paged=False, scale=1.0 / 16,
                                nan_tail=nan_tail, name="c1")
    if n == 2:
        return make_decode_case(seed, batch=64, ctx_lens=[4096] * 64, hq=64, hkv=1, d=256,
                                kv_format="bf16", paged=True, scale=1.0 / 16,
                                nan_tail=nan_tail, name="c2")
    if n == 3:
        return make_decode_case(seed, batch=128, ctx_lens=ragged_lengths(128), hq=64, hkv=1,
                                d=256, kv_format="bf16", paged=True, scale=1.0 / 16,
                                nan_tail=nan_tail, name="c3")
    if n == 4:
        return make_decode_case(seed, batch=256, ctx_lens=[4096] * 256, hq=64, hkv=1, d=256,
                                kv_format="e4m3", q_format="bf16", paged=True,
                                scale=1.0 / 16, nan_tail=nan_tail, draw_q=False, name="c4")
    if n == 5:
        w = 512 if window is None else window
        return make_decode_case(seed, batch=32, ctx_lens=[32768] * 32, hq=64, hkv=4, d=192,
                                kv_format="bf16", paged=True, scale=1.0 / np.sqrt(192),
                                window=w, nan_tail=nan_tail, name="c5")
    raise ValueError(f"no config {n}")


def config_query_inputs(seed=4, *, batch=256):
    """Config 4's query-path inputs, from the generator ``default_rng([seed, 1])``
    in the order x, W_qdown, W_qup."""
    rng = np.random.default_rng([seed, 1])
    return make_query_inputs(rng, batch=batch)
