"""Shared helpers for GPU parity tests: move generator cases to the device, run
the library through its binding, and compare with the oracle."""

import numpy as np
import torch

import decode_attention_mfa_amd as mfa
from workloads.torch_io import raw_to_tensor as _raw_to_tensor, to_device  # noqa: F401

# Parity bars: bf16 / FP8 inputs -> max-abs 2e-2 and rel-L2 5e-3; fp32 -> 1e-4.
TOL = {"bf16": (2e-2, 5e-3), "e4m3": (2e-2, 5e-3), "f32": (1e-4, 1e-4)}


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


def assert_parity(got, ref, fmt, what="", per_slot=False):
    """Whole-tensor max-abs and relative-L2 within the bar of ``fmt``; with
    per_slot, every slot (leading index) must also meet it on its own.  The
    message names the worst slot."""
    max_abs_tol, rel_tol = TOL[fmt]
    g = got.detach().float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    max_abs, rel_l2 = errors(got, ref)
    gg = g.astype(np.float64).reshape(g.shape[0], -1)
    rr = np.asarray(ref, dtype=np.float64).reshape(g.shape[0], -1)
    slot_abs = np.abs(gg - rr).max(axis=1) if gg.size else np.zeros(0)
    norms = np.linalg.norm(rr, axis=1)
    slot_rel = np.linalg.norm(gg - rr, axis=1) / np.where(norms > 0, norms, 1.0)
    worst = int(np.argmax(slot_rel)) if len(slot_rel) else -1
    msg = (f"{what}: max_abs={max_abs:.3e} (tol {max_abs_tol}) rel_l2={rel_l2:.3e} (tol {rel_tol}); "
           f"worst slot {worst}: max_abs={slot_abs[worst] if worst >= 0 else 0:.3e} "
           f"rel_l2={slot_rel[worst] if worst >= 0 else 0:.3e}")
    assert max_abs <= max_abs_tol and rel_l2 <= rel_tol, msg
    if per_slot:
        assert np.all(slot_abs <= max_abs_tol) and np.all(slot_rel <= rel_tol), msg
    return max_abs, rel_l2
