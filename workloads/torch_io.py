"""Move generator cases into torch device tensors (data movement only).

The raw storage arrays of :mod:`workloads.gen` (bf16 bit patterns, E4M3 codes,
float32 values, int32 tables and lengths) are copied bit for bit into device
tensors of the matching torch dtype.  Nothing here computes anything of the
method; it serves the benchmark and the tests alike.
"""

import numpy as np


def raw_to_tensor(arr, fmt, device):
    """A device tensor holding the raw storage array ``arr`` of format ``fmt``
    ("bf16" bits, "e4m3" codes or "f32" values), bit for bit."""
    import torch
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if fmt == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).to(device)
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    raise ValueError(fmt)


def to_device(case, device="cuda", out_format=None):
    """The tensors of one decode call: q, k, v, table, lens, k_scale, v_scale and
    an output filled with NaN (so that an unwritten element shows)."""
    import torch
    out_format = out_format or case.out_format
    t = {
        "q": raw_to_tensor(case.q, case.q_format, device) if case.q is not None else None,
        "k": raw_to_tensor(case.k_cache, case.kv_format, device),
        "v": raw_to_tensor(case.v_cache, case.kv_format, device),
        "table": (torch.from_numpy(case.block_table).to(device)
                  if case.block_table is not None else None),
        "lens": torch.from_numpy(case.ctx_lens.astype(np.int32)).to(device),
        "k_scale": (torch.from_numpy(case.k_scale).to(device) if case.k_scale is not None else None),
        "v_scale": (torch.from_numpy(case.v_scale).to(device) if case.v_scale is not None else None),
    }
    odt = torch.float32 if out_format == "f32" else torch.bfloat16
    t["out"] = torch.full((case.batch, case.hq, case.d), float("nan"), dtype=odt, device=device)
    return t
