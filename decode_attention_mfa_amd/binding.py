"""Thin PyTorch binding over the C ABI: argument marshalling only.

Each function reads shapes, dtypes, data pointers and the current stream from
torch tensors, fills the descriptor and calls the library entry point of the
same name.  Every step of the computation runs in the HIP kernels.  A missing
library raises (decode_attention_mfa_amd._lib.LibraryNotBuilt).

Workspaces: pass `workspace=` (a uint8 CUDA tensor, 256-byte aligned) to keep
calls allocation-free (e.g. under graph capture); otherwise a per-device
workspace is grown on demand and reused, so calls that use the default
workspace must be ordered on one stream.
"""

import ctypes

import torch

from . import _lib
from ._lib import (MFA_BF16, MFA_F32, MFA_FP8_E4M3, MfaDecodeDesc, MfaKvAppendDesc,
                   MfaQueryProjDesc, MfaSparseDesc, check)

PAGE = 64
_workspaces = {}


def _dtype_code(t, allow_fp8=False):
    if t.dtype == torch.float32:
        return MFA_F32
    if t.dtype == torch.bfloat16:
        return MFA_BF16
    if allow_fp8 and t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MFA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    """Data pointer of a tensor the library reads or writes as a dense
    row-major array; a strided view would be read with the wrong strides."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(device, nbytes, given, kind):
    """A cached per-device workspace of at least nbytes, one per kind."""
    if nbytes == 0:
        return given, 0 if given is None else given.numel()
    if given is not None:
        return given, given.numel()
    key = (device.index if device.index is not None else torch.cuda.current_device(), kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes + 256:
        ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    off = (-ws.data_ptr()) % 256
    return ws[off:], ws.numel() - off


def decode_desc(q, k_cache, block_table, out, num_splits=0):
    """Build an MfaDecodeDesc from tensors (paged when block_table is given)."""
    B, hq, d = q.shape
    if block_table is not None:
        hkv = k_cache.shape[1]
        max_blocks = block_table.shape[1]
        num_blocks = k_cache.shape[0]
    else:
        hkv = k_cache.shape[2]
        if k_cache.shape[1] % PAGE:
            raise ValueError(f"a contiguous cache's capacity ({k_cache.shape[1]}) must be a "
                             f"multiple of {PAGE} tokens")
        max_blocks = k_cache.shape[1] // PAGE
        num_blocks = 0
    return MfaDecodeDesc(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=PAGE,
                         max_blocks_per_seq=max_blocks, num_blocks=num_blocks,
                         q_dtype=_dtype_code(q), kv_dtype=_dtype_code(k_cache, allow_fp8=True),
                         out_dtype=_dtype_code(out), num_splits=int(num_splits))


def mfa_decode_workspace_size(desc, window=0):
    return int(_lib.load().mfa_decode_workspace_size(ctypes.byref(desc), int(window)))


def mfa_decode_plan_splits(desc, window=0, num_cus=256):
    return int(_lib.load().mfa_decode_plan_splits(ctypes.byref(desc), int(window), int(num_cus)))


# Descriptor and workspace size per call shape: a decode loop calls with the
# same shapes every step, so the marshalling cost is paid once.
_plans = {}


def _plan(q, k_cache, block_table, out, num_splits, window):
    key = (tuple(q.shape), q.dtype, tuple(k_cache.shape), k_cache.dtype,
           None if block_table is None else tuple(block_table.shape), out.dtype,
           int(num_splits), int(window), q.device.index)
    plan = _plans.get(key)
    if plan is None:
        desc = decode_desc(q, k_cache, block_table, out, num_splits)
        plan = (desc, ctypes.byref(desc), mfa_decode_workspace_size(desc, window))
        _plans[key] = plan
    return plan


# V pool layouts (mfa_v_layout in the header).
V_LAYOUTS = {"channel": 0, "subblock8": 1}


def _v_layout_code(v_layout, k_cache, v_cache, block_table):
    """The mfa_v_layout code of a layout name, after checking that v_cache has
    that layout's shape for the K pool it comes with."""
    if v_layout not in V_LAYOUTS:
        raise ValueError(f"v_layout must be one of {sorted(V_LAYOUTS)}, not {v_layout!r}")
    if v_layout == "subblock8":
        if block_table is not None:
            nb, hkv, _, d = k_cache.shape
            want = (nb, hkv, PAGE // 8, d, 8)
        else:
            B, cap, hkv, d = k_cache.shape
            want = (B, hkv, cap // 8, d, 8)
        if tuple(v_cache.shape) != want:
            raise ValueError(f"a sub-blocked V pool must have shape {want}, "
                             f"not {tuple(v_cache.shape)}")
    return V_LAYOUTS[v_layout]


def _decode(entry, q, k_cache, v_cache, block_table, ctx_lens, out, scale, k_scale, v_scale,
            window, num_splits, workspace, stream, v_layout="channel"):
    lib = _lib.load()
    layout = _v_layout_code(v_layout, k_cache, v_cache, block_table)
    _, desc_ref, need = _plan(q, k_cache, block_table, out, num_splits, window)
    ws, ws_bytes = _workspace(q.device, need, workspace, "decode")
    args = [desc_ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(ctx_lens), _ptr(k_scale), _ptr(v_scale), _ptr(out), ctypes.c_float(scale)]
    if entry == "gqa" and layout != V_LAYOUTS["channel"]:
        status = lib.mfa_decode_attention_gqa_layout(*args, ctypes.c_int32(int(window)),
                                                     ctypes.c_int32(layout), _ptr(ws),
                                                     ctypes.c_size_t(ws_bytes), _stream(q, stream))
    elif entry == "gqa":
        args.append(ctypes.c_int32(int(window)))
        status = lib.mfa_decode_attention_gqa(*args, _ptr(ws), ctypes.c_size_t(ws_bytes),
                                              _stream(q, stream))
    else:
        status = lib.mfa_decode_attention(*args, _ptr(ws), ctypes.c_size_t(ws_bytes),
                                          _stream(q, stream))
    check(status)
    return out


def mfa_decode_attention(q, k_cache, v_cache, block_table, ctx_lens, out, scale, *,
                         k_scale=None, v_scale=None, num_splits=0, workspace=None, stream=None):
    """MFA (MQA, one KV head) decode attention; see mfa_decode_attention in the header."""
    return _decode("mqa", q, k_cache, v_cache, block_table, ctx_lens, out, scale, k_scale,
                   v_scale, 0, num_splits, workspace, stream)


def mfa_decode_attention_noalloc(q, k_cache, v_cache, block_table, ctx_lens, out, scale, *,
                                 k_scale=None, v_scale=None, num_splits=0, stream=None):
    """mfa_decode_attention with the library's own per-GPU scratch instead of a
    workspace (no allocation anywhere in the call); see
    mfa_decode_attention_noalloc in the header."""
    lib = _lib.load()
    _, desc_ref, _ = _plan(q, k_cache, block_table, out, num_splits, 0)
    check(lib.mfa_decode_attention_noalloc(desc_ref, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_table), _ptr(ctx_lens), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(out), ctypes.c_float(scale),
                                           _stream(q, stream)))
    return out


def mfa_decode_attention_phase(q, k_cache, v_cache, block_table, ctx_lens, out, scale, phase, *,
                               k_scale=None, v_scale=None, num_splits=0, workspace=None,
                               stream=None):
    """One of the two launches of mfa_decode_attention (1: attention, 2: merge);
    see mfa_decode_attention_phase in the header."""
    lib = _lib.load()
    _, desc_ref, need = _plan(q, k_cache, block_table, out, num_splits, 0)
    ws, ws_bytes = _workspace(q.device, need, workspace, "decode")
    check(lib.mfa_decode_attention_phase(desc_ref, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(block_table), _ptr(ctx_lens), _ptr(k_scale),
                                         _ptr(v_scale), _ptr(out), ctypes.c_float(scale), _ptr(ws),
                                         ctypes.c_size_t(ws_bytes), ctypes.c_int32(int(phase)),
                                         _stream(q, stream)))
    return out


def mfa_decode_attention_gqa(q, k_cache, v_cache, block_table, ctx_lens, out, scale, *,
                             window=0, k_scale=None, v_scale=None, num_splits=0, workspace=None,
                             stream=None, v_layout="channel"):
    """GQA / sliding-window decode attention; see mfa_decode_attention_gqa (and
    mfa_decode_attention_gqa_layout for v_layout="subblock8")."""
    return _decode("gqa", q, k_cache, v_cache, block_table, ctx_lens, out, scale, k_scale,
                   v_scale, window, num_splits, workspace, stream, v_layout)


def mfa_decode_mtp_workspace_size(desc, num_query_tokens):
    return int(_lib.load().mfa_decode_mtp_workspace_size(ctypes.byref(desc),
                                                         int(num_query_tokens)))


def mfa_decode_attention_mtp(q, k_cache, v_cache, block_table, ctx_lens, out, scale, *,
                             k_scale=None, v_scale=None, num_splits=0, workspace=None,
                             stream=None):
    """Multi-token queries per slot: q and out [B, Tq, Hq, d], ctx_lens counting
    all Tq new tokens; see mfa_decode_attention_mtp in the header."""
    lib = _lib.load()
    B, tq, hq, d = q.shape
    key = ("mtp", tuple(q.shape), q.dtype, tuple(k_cache.shape), k_cache.dtype,
           None if block_table is None else tuple(block_table.shape), out.dtype,
           int(num_splits), q.device.index)
    plan = _plans.get(key)
    if plan is None:
        desc = decode_desc(q[:, 0], k_cache, block_table, out[:, 0], num_splits)   # B sequences
        plan = (desc, ctypes.byref(desc), mfa_decode_mtp_workspace_size(desc, tq))
        _plans[key] = plan
    _, desc_ref, need = plan
    ws, ws_bytes = _workspace(q.device, need, workspace, "decode")
    check(lib.mfa_decode_attention_mtp(desc_ref, ctypes.c_int32(tq), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens),
                                       _ptr(k_scale), _ptr(v_scale), _ptr(out),
                                       ctypes.c_float(scale), _ptr(ws), ctypes.c_size_t(ws_bytes),
                                       _stream(q, stream)))
    return out


def kv_append_desc(k_new, k_cache, block_table):
    """Build an MfaKvAppendDesc from tensors (paged when block_table is given)."""
    B, hkv, d = k_new.shape
    if block_table is not None:
        max_blocks, num_blocks = block_table.shape[1], k_cache.shape[0]
    else:
        if k_cache.shape[1] % PAGE:
            raise ValueError(f"a contiguous cache's capacity ({k_cache.shape[1]}) must be a "
                             f"multiple of {PAGE} tokens")
        max_blocks, num_blocks = k_cache.shape[1] // PAGE, 0
    return MfaKvAppendDesc(batch=B, num_kv_heads=hkv, head_dim=d, page_size=PAGE,
                           max_blocks_per_seq=max_blocks, num_blocks=num_blocks,
                           new_dtype=_dtype_code(k_new),
                           kv_dtype=_dtype_code(k_cache, allow_fp8=True))


def mfa_kv_append(k_new, v_new, k_cache, v_cache, block_table, ctx_lens, *, k_scale=None,
                  v_scale=None, active=None, stream=None, v_layout="channel"):
    """Append one token's K/V per slot and advance ctx_lens on the device; see
    mfa_kv_append (and mfa_kv_append_layout for v_layout="subblock8")."""
    lib = _lib.load()
    layout = _v_layout_code(v_layout, k_cache, v_cache, block_table)
    desc = kv_append_desc(k_new, k_cache, block_table)
    args = [ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), _ptr(ctx_lens), _ptr(k_scale), _ptr(v_scale), _ptr(active)]
    if layout != V_LAYOUTS["channel"]:
        check(lib.mfa_kv_append_layout(*args, ctypes.c_int32(layout), _stream(k_new, stream)))
    else:
        check(lib.mfa_kv_append(*args, _stream(k_new, stream)))


def sparse_desc(batch, block_table, k_cache, out, num_splits=0):
    return MfaSparseDesc(batch=batch, max_blocks_per_seq=block_table.shape[1],
                         num_blocks=k_cache.shape[0] if k_cache is not None else 0,
                         out_dtype=_dtype_code(out) if out is not None else MFA_BF16,
                         num_splits=int(num_splits))


def mfa_sparse_summarize(k_idx, z, ctx_lens, summaries, *, block_table, stream=None):
    """Block summaries of the complete 8-token blocks; see mfa_sparse_summarize."""
    lib = _lib.load()
    desc = sparse_desc(k_idx.shape[0], block_table, None, None)
    check(lib.mfa_sparse_summarize(ctypes.byref(desc), _ptr(k_idx), _ptr(z), _ptr(ctx_lens),
                                   _ptr(summaries), _stream(k_idx, stream)))
    return summaries


def mfa_sparse_summarize_new(k_idx, z, ctx_lens, summaries, new_tokens, *, block_table,
                             stream=None):
    """Summaries of only the blocks the last new_tokens tokens completed; see
    mfa_sparse_summarize_new."""
    lib = _lib.load()
    desc = sparse_desc(k_idx.shape[0], block_table, None, None)
    check(lib.mfa_sparse_summarize_new(ctypes.byref(desc), _ptr(k_idx), _ptr(z), _ptr(ctx_lens),
                                       ctypes.c_int32(int(new_tokens)), _ptr(summaries),
                                       _stream(k_idx, stream)))
    return summaries


def mfa_sparse_select(q_idx, w, summaries, ctx_lens, selected, num_selected, *, block_table,
                      workspace=None, stream=None):
    """Weighted-ReLU scores and the causal top-512; see mfa_sparse_select."""
    lib = _lib.load()
    desc = sparse_desc(q_idx.shape[0], block_table, None, None)
    need = int(lib.mfa_sparse_workspace_size(ctypes.byref(desc)))
    ws, ws_bytes = _workspace(q_idx.device, need, workspace, "sparse")
    check(lib.mfa_sparse_select(ctypes.byref(desc), _ptr(q_idx), _ptr(w), _ptr(summaries),
                                _ptr(ctx_lens), _ptr(selected), _ptr(num_selected), _ptr(ws),
                                ctypes.c_size_t(ws_bytes), _stream(q_idx, stream)))
    return selected, num_selected


def mfa_sparse_attention(q, k_cache, v_cache, block_table, ctx_lens, selected, num_selected, out,
                         scale, *, num_splits=0, workspace=None, stream=None):
    """Attention over the selected blocks and the current block; see
    mfa_sparse_attention."""
    lib = _lib.load()
    desc = sparse_desc(q.shape[0], block_table, k_cache, out, num_splits)
    need = int(lib.mfa_sparse_workspace_size(ctypes.byref(desc)))
    ws, ws_bytes = _workspace(q.device, need, workspace, "sparse")
    check(lib.mfa_sparse_attention(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(ctx_lens), _ptr(selected),
                                   _ptr(num_selected), _ptr(out), ctypes.c_float(scale), _ptr(ws),
                                   ctypes.c_size_t(ws_bytes), _stream(q, stream)))
    return out


def query_proj_desc(x, w_qup, q_out, num_heads, eps):
    B, hidden = x.shape
    rank = w_qup.shape[1]
    width = w_qup.shape[0]
    return MfaQueryProjDesc(batch=B, hidden=hidden, rank=rank, num_heads=num_heads,
                            head_dim=width // num_heads, eps=float(eps),
                            out_dtype=_dtype_code(q_out))


def mfa_query_proj(x, w_qdown, w_qup, q_out, *, num_heads=64, gain=None, eps=1e-6,
                   workspace=None, stream=None):
    """Low-rank query path; weights in [out, in] layout; see mfa_query_proj."""
    lib = _lib.load()
    desc = query_proj_desc(x, w_qup, q_out, num_heads, eps)
    need = int(lib.mfa_query_proj_workspace_size(ctypes.byref(desc)))
    ws, ws_bytes = _workspace(x.device, need, workspace, "query_proj")
    check(lib.mfa_query_proj(ctypes.byref(desc), _ptr(x), _ptr(w_qdown), _ptr(w_qup),
                             _ptr(gain), _ptr(q_out), _ptr(ws), ctypes.c_size_t(ws_bytes),
                             _stream(x, stream)))
    return q_out


def mfa_stream_read(src, sink, *, stream=None):
    """Read-rate reference: streams every byte of the CUDA tensor `src` once
    (see mfa_stream_read in the header); `sink` is an int32 CUDA tensor of at
    least num_cus * 512 entries, whose XOR equals the XOR of src's words."""
    lib = _lib.load()
    if sink.dtype != torch.int32:
        raise TypeError("sink must be int32")
    check(lib.mfa_stream_read(_ptr(src), ctypes.c_size_t(src.numel() * src.element_size()),
                              _ptr(sink), ctypes.c_size_t(sink.numel()), _stream(src, stream)))
    return sink
