"""Seeded synthetic decode-attention inputs drawn on the GPU, for shapes whose
host generation would take minutes (gigabyte KV pools).

Recipe (one ``torch.Generator`` on the device, ``manual_seed(seed)``), fixed draw
order: q -> K pool -> V pool -> pool permutation.  Values are N(0, 1) drawn
in float32 and rounded to bf16 by torch's round-to-nearest-even cast; for an
E4M3 cache each KV head gets one fp32 scale = absmax / 448 over its valid
entries and the codes are torch's float8_e4m3fn cast of x / scale (clipped
to +-448), as in the host recipe.  The
pool is drawn directly in physical order, and logical block k of the
(slot, block) order sits at pool position ``perm[k]``; every block is an iid
draw, so the value distribution is the host recipe's (:mod:`workloads.gen`),
but the values differ.  Tail rows past each slot's length hold NaN
(bf16 0x7FC0, E4M3 0x7F) when ``nan_tail`` is set; unused table entries are -1.

Like :mod:`workloads.gen`, this module only draws and lays out numbers: it
holds none of the attention arithmetic.  :meth:`DeviceCase.host_slots`
copies the blocks of a few slots back into a compact host
:class:`~workloads.gen.DecodeCase`, which the oracle evaluates.
"""

from dataclasses import dataclass

import numpy as np

from .gen import E4M3_MAX, E4M3_NAN, PAGE, DecodeCase


@dataclass
class DeviceCase:
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    d: int
    scale: float
    window: int
    ctx_lens: np.ndarray        # [B] int32 (host copy)
    block_table: np.ndarray     # [B, M] int32 (host copy)
    q: "object"                 # torch bf16 [B, Hq, d]
    k: "object"                 # torch bf16 [num_blocks, Hkv, P, d]
    v: "object"                 # torch bf16 [num_blocks, Hkv, d, P]
    table: "object"             # torch int32 [B, M]
    lens: "object"              # torch int32 [B]
    kv_format: str = "bf16"     # "bf16" | "e4m3"
    k_scale: "object" = None    # torch fp32 [Hkv] (e4m3)
    v_scale: "object" = None
    q_format: str = "bf16"
    out_format: str = "bf16"

    def host_slots(self, slots):
        """The given slots as a host DecodeCase (raw bf16 bits) holding only
        their blocks, renumbered; slot i of the result is ``slots[i]``."""
        import torch
        slots = [int(s) for s in slots]
        nb = [(int(self.ctx_lens[s]) + PAGE - 1) // PAGE for s in slots]
        width = max(max(nb), 1)
        ids = []
        table = np.full((len(slots), width), -1, dtype=np.int32)
        for i, s in enumerate(slots):
            for j in range(nb[i]):
                table[i, j] = len(ids)
                ids.append(int(self.block_table[s, j]))
        if not ids:
            ids = [0]
        idx = torch.as_tensor(ids, dtype=torch.long, device=self.k.device)

        def raw(t):
            t = t.index_select(0, idx)
            if self.kv_format == "e4m3":
                return t.view(torch.uint8).cpu().numpy()
            return t.view(torch.int16).cpu().numpy().view(np.uint16)

        sidx = torch.as_tensor(slots, dtype=torch.long, device=self.q.device)
        q = self.q.index_select(0, sidx).view(torch.int16).cpu().numpy().view(np.uint16)
        ks = self.k_scale.cpu().numpy() if self.k_scale is not None else None
        vs = self.v_scale.cpu().numpy() if self.v_scale is not None else None
        return DecodeCase(name=f"{self.name}[{slots}]", seed=self.seed, batch=len(slots),
                          hq=self.hq, hkv=self.hkv, d=self.d, q_format="bf16",
                          kv_format=self.kv_format, out_format=self.out_format, q=q,
                          k_cache=raw(self.k), v_cache=raw(self.v),
                          ctx_lens=self.ctx_lens[slots].astype(np.int32), block_table=table,
                          scale=self.scale, window=self.window, k_scale=ks, v_scale=vs)


def make_device_case(seed, *, batch, ctx_lens, hq, hkv, d, window=0, scale=None,
                     kv_format="bf16", nan_tail=True, device="cuda", name="device",
                     chunk_blocks=2048):
    """A paged bf16 or E4M3 case drawn on ``device``."""
    import torch
    lens = np.asarray(ctx_lens, dtype=np.int64)
    if lens.shape != (batch,):
        raise ValueError("ctx_lens must have one entry per slot")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    nblk_slot = (lens + PAGE - 1) // PAGE
    nblk = max(int(nblk_slot.sum()), 1)
    width = max(int(nblk_slot.max()) if batch else 1, 1)

    q = torch.randn((batch, hq, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    fp8 = kv_format == "e4m3"
    if kv_format not in ("bf16", "e4m3"):
        raise ValueError(kv_format)
    draw_dtype = torch.float32 if fp8 else torch.bfloat16
    k = torch.empty((nblk, hkv, PAGE, d), dtype=draw_dtype, device=device)
    v = torch.empty((nblk, hkv, d, PAGE), dtype=draw_dtype, device=device)
    for pool in (k, v):
        for s in range(0, nblk, chunk_blocks):
            e = min(nblk, s + chunk_blocks)
            pool[s:e] = torch.randn(pool[s:e].shape, generator=g, device=device,
                                    dtype=torch.float32).to(draw_dtype)
    perm = torch.randperm(nblk, generator=g, device=device).cpu().numpy().astype(np.int32)

    table = np.full((batch, width), -1, dtype=np.int32)
    tails = []                                   # (pool block, first invalid row)
    kk = 0
    for b in range(batch):
        for i in range(int(nblk_slot[b])):
            table[b, i] = perm[kk]
            tail = int(lens[b]) - i * PAGE
            if tail < PAGE:
                tails.append((int(perm[kk]), tail))
            kk += 1
    k_scale = v_scale = None
    if fp8:
        for blk, tail in tails:                  # scales over valid entries only
            k[blk, :, tail:, :] = 0
            v[blk, :, :, tail:] = 0
        k_scale = k.abs().amax(dim=(0, 2, 3)) / E4M3_MAX
        v_scale = v.abs().amax(dim=(0, 2, 3)) / E4M3_MAX
        k = (k / k_scale.view(1, -1, 1, 1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        v = (v / v_scale.view(1, -1, 1, 1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    if nan_tail:
        for blk, tail in tails:
            if fp8:
                k.view(torch.uint8)[blk, :, tail:, :] = int(E4M3_NAN)
                v.view(torch.uint8)[blk, :, :, tail:] = int(E4M3_NAN)
            else:
                k[blk, :, tail:, :] = float("nan")
                v[blk, :, :, tail:] = float("nan")
    return DeviceCase(name=name, seed=seed, batch=batch, hq=hq, hkv=hkv, d=d,
                      scale=float(scale), window=int(window),
                      ctx_lens=lens.astype(np.int32), block_table=table, q=q, k=k, v=v,
                      table=torch.from_numpy(table).to(device),
                      lens=torch.from_numpy(lens.astype(np.int32)).to(device),
                      kv_format=kv_format, k_scale=k_scale, v_scale=v_scale)
