"""Shared helpers for GPU parity tests: move generator cases to the device, run
the library through its binding, and compare with the oracle."""

import numpy as np
import torch

import decode_attention_mfa_amd as mfa

# Parity bars: bf16 / FP8 inputs -> max-abs 2e-2 and rel-L2 5e-3; fp32 -> 1e-4.
TOL = {"bf16": (2e-2, 5e-3), "e4m3": (2e-2, 5e-3), "f32": (1e-4, 1e-4)}


def _raw_to_tensor(arr, fmt, device):
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    if fmt == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).to(device)
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    raise ValueError(fmt)


def to_device(case, device="cuda", out_format=None):
    out_format = out_format or case.out_format
    t = {
        "q": _raw_to_tensor(case.q, case.q_format, device) if case.q is not None else None,
        "k": _raw_to_tensor(case.k_cache, case.kv_format, device),
        "v": _raw_to_tensor(case.v_cache, case.kv_format, device),
        "table": (torch.from_numpy(case.block_table).to(device)
                  if case.block_table is not None else None),
        "lens": torch.from_numpy(case.ctx_lens.astype(np.int32)).to(device),
        "k_scale": (torch.from_numpy(case.k_scale).to(device) if case.k_scale is not None else None),
        "v_scale": (torch.from_numpy(case.v_scale).to(device) if case.v_scale is not None else None),
    }
    odt = torch.float32 if out_format == "f32" else torch.bfloat16
    t["out"] = torch.full((case.batch, case.hq, case.d), float("nan"), dtype=odt, device=device)
    return t


def run_decode(case, t, *, num_splits=0, window=None, q=None, lens=None, table=None):
    """Run the library on a device case; MQA entry when Hkv == 1 and no window."""
    w = case.window if window is None else window
    args = (t["q"] if q is None else q, t["k"], t["v"], t["table"] if table is None else table,
            t["lens"] if lens is None else lens, t["out"], case.scale)
    if case.hkv == 1 and w == 0:
        mfa.mfa_decode_attention(*args, k_scale=t["k_scale"], v_scale=t["v_scale"],
                                 num_splits=num_splits)
    else:
        mfa.mfa_decode_attention_gqa(*args, window=w, k_scale=t["k_scale"],
                                     v_scale=t["v_scale"], num_splits=num_splits)
    torch.cuda.synchronize()
    return t["out"]


def errors(got, ref):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    diff = np.abs(g - ref)
    max_abs = float(np.max(diff)) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(g - ref) / denom) if denom > 0 else float(np.linalg.norm(g - ref))
    return max_abs, rel_l2


def assert_parity(got, ref, fmt, what=""):
    max_abs_tol, rel_tol = TOL[fmt]
    g = got.detach().float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    max_abs, rel_l2 = errors(got, ref)
    assert max_abs <= max_abs_tol and rel_l2 <= rel_tol, (
        f"{what}: max_abs={max_abs:.3e} (tol {max_abs_tol}) rel_l2={rel_l2:.3e} (tol {rel_tol})")
    return max_abs, rel_l2
