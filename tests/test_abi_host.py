"""CPU-only tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host-side validation / planning behaves as documented.  No
call here reaches a kernel launch (every call either fails validation first or
is a pure planning query)."""

import ctypes
import os
import re

import pytest

from decode_attention_mfa_amd import _lib
from decode_attention_mfa_amd._lib import MFA_BF16, MFA_F32, MFA_FP8_E4M3, MfaDecodeDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")

MFA_ERR_NULL, MFA_ERR_DTYPE, MFA_ERR_SHAPE, MFA_ERR_ALIGN = 1, 2, 3, 4
MFA_ERR_ARG, MFA_ERR_WORKSPACE = 5, 6


def header_symbols():
    text = open(os.path.join(ROOT, "include", "mfa_decode.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(mfa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_what_binding_lists():
    assert header_symbols() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in header_symbols():
        assert hasattr(lib, name), name
    assert lib.mfa_abi_version() == 1
    for s in range(8):
        assert lib.mfa_status_string(s)


def desc(**kw):
    d = dict(batch=64, num_q_heads=64, num_kv_heads=1, head_dim=256, page_size=64,
             max_blocks_per_seq=64, num_blocks=4096, q_dtype=MFA_BF16, kv_dtype=MFA_BF16,
             out_dtype=MFA_BF16, num_splits=4)
    d.update(kw)
    return MfaDecodeDesc(**d)


# 16-byte aligned fake addresses: validation never dereferences them.
A = ctypes.c_void_p(0x10000)


def call_mqa(d, q=A, k=A, v=A, table=A, lens=A, ks=None, vs=None, out=A, scale=0.0625,
             ws=None, ws_bytes=0):
    lib = _lib.load()
    return lib.mfa_decode_attention(ctypes.byref(d) if d is not None else None, q, k, v, table,
                                    lens, ks, vs, out, ctypes.c_float(scale), ws,
                                    ctypes.c_size_t(ws_bytes), None)


def call_gqa(d, window, **kw):
    lib = _lib.load()
    return lib.mfa_decode_attention_gqa(ctypes.byref(d), A, A, A, A, A, None, None, A,
                                        ctypes.c_float(0.07), ctypes.c_int32(window), None,
                                        ctypes.c_size_t(0), None)


def test_null_descriptor_and_pointers():
    assert call_mqa(None) == MFA_ERR_NULL
    assert call_mqa(desc(), q=None) == MFA_ERR_NULL
    assert call_mqa(desc(), out=None) == MFA_ERR_NULL
    assert call_mqa(desc(), lens=None) == MFA_ERR_NULL
    # FP8 needs both scales
    assert call_mqa(desc(kv_dtype=MFA_FP8_E4M3), ks=A, vs=None) == MFA_ERR_NULL
    assert call_mqa(desc(kv_dtype=MFA_FP8_E4M3), ks=None, vs=A) == MFA_ERR_NULL


def test_dtype_combinations():
    assert call_mqa(desc(q_dtype=MFA_F32)) == MFA_ERR_DTYPE            # bf16 kv needs bf16 q
    assert call_mqa(desc(out_dtype=MFA_FP8_E4M3)) == MFA_ERR_DTYPE
    assert call_mqa(desc(kv_dtype=MFA_F32)) == MFA_ERR_DTYPE           # f32 kv needs f32 q/out
    assert call_mqa(desc(kv_dtype=7)) == MFA_ERR_DTYPE


def test_shape_rules():
    assert call_mqa(desc(num_kv_heads=2, num_q_heads=128)) == MFA_ERR_SHAPE   # MQA entry: Hkv == 1
    assert call_mqa(desc(page_size=32)) == MFA_ERR_SHAPE
    assert call_mqa(desc(head_dim=128)) == MFA_ERR_SHAPE                      # not (64, 256)
    assert call_mqa(desc(max_blocks_per_seq=0)) == MFA_ERR_SHAPE
    assert call_mqa(desc(batch=-1)) == MFA_ERR_SHAPE
    assert call_mqa(desc(num_splits=-2)) == MFA_ERR_SHAPE
    assert call_gqa(desc(num_q_heads=64, num_kv_heads=3), 0) == MFA_ERR_SHAPE  # 64 % 3


def test_fp8_on_the_mfma_paths_only():
    # 16 heads per group reads E4M3 too: it then needs both scales ...
    assert call_gqa(desc(num_q_heads=64, num_kv_heads=4, head_dim=192,
                         kv_dtype=MFA_FP8_E4M3), 0) == MFA_ERR_NULL
    # ... while a shape that only the fp32 kernel serves is refused for E4M3
    assert call_gqa(desc(num_q_heads=64, num_kv_heads=4, head_dim=128,
                         kv_dtype=MFA_FP8_E4M3), 0) == MFA_ERR_SHAPE


def test_alignment_scale_window_workspace():
    assert call_mqa(desc(), q=ctypes.c_void_p(0x10008)) == MFA_ERR_ALIGN
    assert call_mqa(desc(), out=ctypes.c_void_p(0x10004)) == MFA_ERR_ALIGN
    assert call_mqa(desc(), scale=float("nan")) == MFA_ERR_ARG
    assert call_mqa(desc(), scale=float("inf")) == MFA_ERR_ARG
    assert call_gqa(desc(num_kv_heads=4, head_dim=192, num_splits=2), -1) == MFA_ERR_ARG
    # 4 forced splits need a workspace
    assert call_mqa(desc()) == MFA_ERR_WORKSPACE
    assert call_mqa(desc(), ws=A, ws_bytes=16) == MFA_ERR_WORKSPACE
    assert call_mqa(desc(), ws=ctypes.c_void_p(0x10010), ws_bytes=1 << 30) == MFA_ERR_ALIGN


def test_empty_batch_is_a_no_op():
    assert call_mqa(desc(batch=0), q=None, out=None) == 0


def test_workspace_size_matches_partials():
    lib = _lib.load()
    d = desc(num_splits=4)
    rows = 64 * 1 * 4 * 64
    expect_o = rows * 256 * 4
    got = lib.mfa_decode_workspace_size(ctypes.byref(d), 0)
    assert got >= expect_o + rows * 8 and got % 256 == 0
    assert lib.mfa_decode_workspace_size(ctypes.byref(desc(num_splits=1)), 0) == 0


@pytest.mark.parametrize("batch,blocks,cus,window,expect", [
    (64, 64, 256, 0, 4),       # B=64 x 4K: one workgroup per compute unit
    (256, 64, 256, 0, 1),      # B=256 x 4K: no split needed
    (1, 64, 256, 0, 16),       # one slot: 16 chunks of 4 pages
    (2, 2, 256, 0, 1),         # tiny context: chunks never below 4 pages
    # A split must save >= 448 KB of bf16 K/V per workgroup:
    (32, 512, 256, 512, 1),    # 512-key window, <= 9 pages: 2 chunks would save 192 KB
    (64, 8, 256, 0, 1),        # B=64 x 512: 2 chunks would save 4 pages = 256 KB
    (64, 12, 256, 0, 3),       # B=64 x 768: 3 chunks of 4 save 8 pages = 512 KB
    (32, 16, 256, 1024, 1),    # GQA 1024-key window: 2 chunks would save 8 x 48 KB
])
def test_split_heuristic(batch, blocks, cus, window, expect):
    lib = _lib.load()
    kv = 1 if window == 0 else 4
    dim = 256 if window == 0 else 192
    d = desc(batch=batch, max_blocks_per_seq=blocks, num_splits=0, num_kv_heads=kv,
             head_dim=dim)
    got = lib.mfa_decode_plan_splits(ctypes.byref(d), window, cus)
    assert got == expect


def test_forced_splits_are_honoured_up_to_the_page_count():
    lib = _lib.load()
    for forced, expect in [(1, 1), (3, 3), (8, 8), (100, 64)]:
        d = desc(num_splits=forced)
        assert lib.mfa_decode_plan_splits(ctypes.byref(d), 0, 256) == expect


def call_mtp(d, tq, ws=None, ws_bytes=0, q=A):
    lib = _lib.load()
    return lib.mfa_decode_attention_mtp(ctypes.byref(d), ctypes.c_int32(tq), q, A, A, A, A,
                                        None, None, A, ctypes.c_float(0.0625), ws,
                                        ctypes.c_size_t(ws_bytes), None)


def test_multi_token_entry_rules():
    lib = _lib.load()
    assert call_mtp(desc(), 0) == MFA_ERR_SHAPE
    assert call_mtp(desc(), 17) == MFA_ERR_SHAPE
    assert call_mtp(desc(num_kv_heads=2, num_q_heads=128), 2) == MFA_ERR_SHAPE   # Hkv == 1
    # fp32 MFA shapes run on the scalar path, which has no multi-token variant
    assert call_mtp(desc(q_dtype=MFA_F32, kv_dtype=MFA_F32, out_dtype=MFA_F32), 2) == MFA_ERR_SHAPE
    assert call_mtp(desc(), 2) == MFA_ERR_WORKSPACE               # forced splits need room
    assert call_mtp(desc(), 2, q=None) == MFA_ERR_NULL
    assert call_mtp(desc(batch=0), 3, q=None) == 0
    # The query slots (batch x Tq/2 token pairs, or batch x Tq single tokens)
    # set the launch grid: a batch inside the 65535 grid-row limit whose
    # slots are not is a shape error, not a launch failure.
    assert call_mtp(desc(batch=40000), 4) == MFA_ERR_SHAPE       # 80000 pair slots
    assert call_mtp(desc(batch=30000), 3) == MFA_ERR_SHAPE       # 90000 single-token slots
    assert call_mtp(desc(batch=32000), 2) == MFA_ERR_WORKSPACE   # 32000 slots: valid shape
    # The workspace of Tq tokens is that of Tq times as many single-token slots.
    for tq in (1, 2, 4):
        got = lib.mfa_decode_mtp_workspace_size(ctypes.byref(desc(num_splits=4)), tq)
        assert got == lib.mfa_decode_workspace_size(ctypes.byref(desc(batch=64 * tq, num_splits=4)), 0)
    assert lib.mfa_decode_mtp_workspace_size(ctypes.byref(desc()), 0) == 0


def sparse(**kw):
    from decode_attention_mfa_amd._lib import MfaSparseDesc
    d = dict(batch=32, max_blocks_per_seq=512, num_blocks=16384, out_dtype=MFA_BF16, num_splits=0)
    d.update(kw)
    return MfaSparseDesc(**d)


def test_sparse_entry_rules():
    lib = _lib.load()
    att = lambda d, ws=None, nbytes=0, q=A: lib.mfa_sparse_attention(
        ctypes.byref(d) if d is not None else None, q, A, A, A, A, A, A, A, ctypes.c_float(0.07),
        ws, ctypes.c_size_t(nbytes), None)
    assert att(None) == MFA_ERR_NULL
    assert att(sparse(out_dtype=MFA_FP8_E4M3)) == MFA_ERR_DTYPE
    assert att(sparse(max_blocks_per_seq=513)) == MFA_ERR_SHAPE         # > 4096 candidate blocks
    # a table width whose candidate count overflows 32 bits is refused, not wrapped
    for wide in (1 << 29, (1 << 31) - 1):
        assert att(sparse(max_blocks_per_seq=wide)) == MFA_ERR_SHAPE
        assert lib.mfa_sparse_workspace_size(ctypes.byref(sparse(max_blocks_per_seq=wide))) == 0
    assert att(sparse(num_splits=66)) == MFA_ERR_SHAPE
    assert att(sparse(num_blocks=0, num_splits=1)) == MFA_ERR_SHAPE
    assert att(sparse(), q=None) == MFA_ERR_NULL
    assert att(sparse(), q=ctypes.c_void_p(0x10008)) == MFA_ERR_ALIGN
    assert att(sparse(num_splits=2)) == MFA_ERR_WORKSPACE
    assert att(sparse(batch=0), q=None) == 0
    assert lib.mfa_sparse_summarize(ctypes.byref(sparse()), None, A, A, A, None) == MFA_ERR_NULL
    assert lib.mfa_sparse_select(ctypes.byref(sparse()), A, A, A, A, A, None, None, 0, None) == MFA_ERR_NULL
    assert lib.mfa_sparse_select(ctypes.byref(sparse()), A, A, A, A, A, A, None, 0, None) == MFA_ERR_WORKSPACE
    # two splits of 33 tiles: partials of 32 x 4 groups x 16 heads x 2 splits
    rows = 32 * 4 * 16 * 2
    got = lib.mfa_sparse_workspace_size(ctypes.byref(sparse(num_splits=2)))
    assert got >= rows * (192 * 4 + 8) and got % 256 == 0
    # one split: the selection's fp32 scores [32, 4, 4096]
    assert lib.mfa_sparse_workspace_size(ctypes.byref(sparse(num_splits=1))) == 32 * 4 * 4096 * 4


def test_phase_entry_rules():
    lib = _lib.load()
    for phase in (0, 3, -1):
        assert lib.mfa_decode_attention_phase(ctypes.byref(desc()), A, A, A, A, A, None, None, A,
                                              ctypes.c_float(0.0625), None, ctypes.c_size_t(0),
                                              ctypes.c_int32(phase), None) == MFA_ERR_ARG
    # forced splits need the workspace in either phase
    for phase in (1, 2):
        assert lib.mfa_decode_attention_phase(ctypes.byref(desc()), A, A, A, A, A, None, None, A,
                                              ctypes.c_float(0.0625), None, ctypes.c_size_t(0),
                                              ctypes.c_int32(phase), None) == MFA_ERR_WORKSPACE


def test_binding_rejects_strided_tensors_and_ragged_capacity():
    # The binding hands the library bare data pointers: a strided view or a
    # contiguous cache whose capacity is not whole 64-token blocks would be
    # read with the wrong layout, so it refuses them before any call.
    import torch
    import decode_attention_mfa_amd as mfa
    q = torch.zeros((2, 64, 256), dtype=torch.bfloat16)
    k = torch.zeros((4, 1, 64, 256), dtype=torch.bfloat16)
    v = torch.zeros((4, 1, 256, 64), dtype=torch.bfloat16)
    table = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.zeros((2,), dtype=torch.int32)
    out = torch.zeros_like(q)
    with pytest.raises(ValueError, match="contiguous"):
        mfa.mfa_decode_attention(q.transpose(1, 2).contiguous().transpose(1, 2), k, v, table,
                                 lens, out, 0.0625, num_splits=1)
    with pytest.raises(ValueError, match="contiguous"):
        mfa.mfa_decode_attention(q, k, v, table.t().contiguous().t(), lens, out, 0.0625,
                                 num_splits=1)
    kc = torch.zeros((2, 100, 1, 256), dtype=torch.bfloat16)      # capacity 100 tokens
    vc = torch.zeros((2, 1, 256, 100), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="multiple of 64"):
        mfa.mfa_decode_attention(q, kc, vc, None, lens, out, 0.0625, num_splits=1)


def test_v_layout_and_incremental_summary_rules():
    from decode_attention_mfa_amd._lib import MfaKvAppendDesc
    lib = _lib.load()

    def gqa_layout(d, layout):
        return lib.mfa_decode_attention_gqa_layout(ctypes.byref(d), A, A, A, A, A, None, None, A,
                                                   ctypes.c_float(0.07), ctypes.c_int32(0),
                                                   ctypes.c_int32(layout), None,
                                                   ctypes.c_size_t(0), None)
    step5 = dict(num_q_heads=64, num_kv_heads=4, head_dim=192, num_splits=1)
    assert gqa_layout(desc(**step5), 2) == MFA_ERR_ARG
    assert gqa_layout(desc(**step5), -1) == MFA_ERR_ARG
    # sub-blocked V is read by the per-group bf16 path only
    assert gqa_layout(desc(num_splits=1), 1) == MFA_ERR_SHAPE                  # MQA shape
    assert gqa_layout(desc(q_dtype=MFA_F32, kv_dtype=MFA_F32, out_dtype=MFA_F32,
                           **step5), 1) == MFA_ERR_SHAPE                       # fp32 path
    lib_fp8 = lib.mfa_decode_attention_gqa_layout(
        ctypes.byref(desc(kv_dtype=MFA_FP8_E4M3, **step5)), A, A, A, A, A, A, A, A,
        ctypes.c_float(0.07), ctypes.c_int32(0), ctypes.c_int32(1), None, ctypes.c_size_t(0), None)
    assert lib_fp8 == MFA_ERR_DTYPE                                            # E4M3 stays channel-major

    def append(kv_dtype, new_dtype, layout):
        d = MfaKvAppendDesc(batch=4, num_kv_heads=4, head_dim=192, page_size=64,
                            max_blocks_per_seq=8, num_blocks=64, new_dtype=new_dtype,
                            kv_dtype=kv_dtype)
        return lib.mfa_kv_append_layout(ctypes.byref(d), A, A, A, A, A, A, A, A, None,
                                        ctypes.c_int32(layout), None)
    assert append(MFA_BF16, MFA_BF16, 3) == MFA_ERR_ARG
    assert append(MFA_F32, MFA_F32, 1) == MFA_ERR_DTYPE
    assert append(MFA_FP8_E4M3, MFA_BF16, 1) == MFA_ERR_DTYPE

    def summ_new(d, n):
        return lib.mfa_sparse_summarize_new(ctypes.byref(d) if d is not None else None, A, A, A,
                                            ctypes.c_int32(n), A, None)
    assert summ_new(None, 1) == MFA_ERR_NULL
    assert summ_new(sparse(), 0) == MFA_ERR_ARG
    assert summ_new(sparse(), -3) == MFA_ERR_ARG
    assert summ_new(sparse(max_blocks_per_seq=4), 4 * 64 + 1) == MFA_ERR_ARG
    assert summ_new(sparse(batch=0), 1) == 0


def test_binding_checks_the_sub_blocked_v_shape():
    import torch
    import decode_attention_mfa_amd as mfa
    q = torch.zeros((2, 64, 192), dtype=torch.bfloat16)
    k = torch.zeros((4, 4, 64, 192), dtype=torch.bfloat16)
    v_channel = torch.zeros((4, 4, 192, 64), dtype=torch.bfloat16)
    table = torch.zeros((2, 2), dtype=torch.int32)
    lens = torch.zeros((2,), dtype=torch.int32)
    out = torch.zeros_like(q)
    with pytest.raises(ValueError, match="sub-blocked V pool"):
        mfa.mfa_decode_attention_gqa(q, k, v_channel, table, lens, out, 0.07, num_splits=1,
                                     v_layout="subblock8")
    with pytest.raises(ValueError, match="v_layout"):
        mfa.mfa_decode_attention_gqa(q, k, v_channel, table, lens, out, 0.07, num_splits=1,
                                     v_layout="tokens")


def test_stream_read_rules():
    """The read-rate reference validates before it launches: NULL pointers,
    a misaligned source and byte counts that are zero or not whole 16-byte
    loads are refused on the host."""
    lib = _lib.load()

    def call(src, nbytes, sink, sink_len):
        return lib.mfa_stream_read(src, ctypes.c_size_t(nbytes), sink, ctypes.c_size_t(sink_len),
                                   None)
    assert call(None, 1 << 20, A, 1 << 20) == MFA_ERR_NULL
    assert call(A, 1 << 20, None, 1 << 20) == MFA_ERR_NULL
    assert call(ctypes.c_void_p(0x10008), 1 << 20, A, 1 << 20) == MFA_ERR_ALIGN
    assert call(A, 0, A, 1 << 20) == MFA_ERR_SHAPE
    assert call(A, (1 << 20) + 8, A, 1 << 20) == MFA_ERR_SHAPE
