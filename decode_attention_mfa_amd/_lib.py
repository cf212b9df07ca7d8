"""ctypes view of the C ABI in include/mfa_decode.h.

Loading fails loudly when the HIP library has not been built: there is no
fallback implementation.
"""

import ctypes
import os

from .build import LIB_PATH

MFA_OK = 0
STATUS_NAMES = {
    0: "MFA_OK", 1: "MFA_ERR_NULL", 2: "MFA_ERR_DTYPE", 3: "MFA_ERR_SHAPE",
    4: "MFA_ERR_ALIGN", 5: "MFA_ERR_ARG", 6: "MFA_ERR_WORKSPACE", 7: "MFA_ERR_LAUNCH",
}
MFA_F32, MFA_BF16, MFA_FP8_E4M3 = 0, 1, 2

# Every symbol the header declares.
EXPORTED = (
    "mfa_decode_attention",
    "mfa_decode_attention_gqa",
    "mfa_decode_attention_gqa_layout",
    "mfa_decode_attention_mtp",
    "mfa_decode_attention_phase",
    "mfa_decode_attention_noalloc",
    "mfa_decode_workspace_size",
    "mfa_decode_mtp_workspace_size",
    "mfa_decode_plan_splits",
    "mfa_kv_append",
    "mfa_kv_append_layout",
    "mfa_query_proj",
    "mfa_query_proj_workspace_size",
    "mfa_sparse_summarize",
    "mfa_sparse_summarize_new",
    "mfa_sparse_select",
    "mfa_sparse_attention",
    "mfa_sparse_workspace_size",
    "mfa_stream_read",
    "mfa_status_string",
    "mfa_abi_version",
)


class MfaDecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


class MfaKvAppendDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("new_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
    ]


class MfaQueryProjDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("out_dtype", ctypes.c_int32),
    ]


class MfaSparseDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("out_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


_LIB = None


class LibraryNotBuilt(RuntimeError):
    pass


def load():
    """Load libmfa_decode.so (once) and declare the signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing: build it with `python -m decode_attention_mfa_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    desc_p = ctypes.POINTER(MfaDecodeDesc)
    qp_p = ctypes.POINTER(MfaQueryProjDesc)
    lib.mfa_decode_attention.argtypes = [desc_p, P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                         ctypes.c_size_t, P]
    lib.mfa_decode_attention.restype = ctypes.c_int
    lib.mfa_decode_attention_gqa.argtypes = [desc_p, P, P, P, P, P, P, P, P, ctypes.c_float,
                                             ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.mfa_decode_attention_gqa.restype = ctypes.c_int
    lib.mfa_decode_attention_gqa_layout.argtypes = [desc_p, P, P, P, P, P, P, P, P, ctypes.c_float,
                                                    ctypes.c_int32, ctypes.c_int32, P,
                                                    ctypes.c_size_t, P]
    lib.mfa_decode_attention_gqa_layout.restype = ctypes.c_int
    lib.mfa_decode_attention_phase.argtypes = [desc_p, P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                               ctypes.c_size_t, ctypes.c_int32, P]
    lib.mfa_decode_attention_phase.restype = ctypes.c_int
    lib.mfa_decode_attention_noalloc.argtypes = [desc_p, P, P, P, P, P, P, P, P, ctypes.c_float, P]
    lib.mfa_decode_attention_noalloc.restype = ctypes.c_int
    lib.mfa_decode_attention_mtp.argtypes = [desc_p, ctypes.c_int32, P, P, P, P, P, P, P, P,
                                             ctypes.c_float, P, ctypes.c_size_t, P]
    lib.mfa_decode_attention_mtp.restype = ctypes.c_int
    lib.mfa_decode_mtp_workspace_size.argtypes = [desc_p, ctypes.c_int32]
    lib.mfa_decode_mtp_workspace_size.restype = ctypes.c_size_t
    lib.mfa_decode_workspace_size.argtypes = [desc_p, ctypes.c_int32]
    lib.mfa_decode_workspace_size.restype = ctypes.c_size_t
    lib.mfa_decode_plan_splits.argtypes = [desc_p, ctypes.c_int32, ctypes.c_int32]
    lib.mfa_decode_plan_splits.restype = ctypes.c_int32
    lib.mfa_stream_read.argtypes = [P, ctypes.c_size_t, P, ctypes.c_size_t, P]
    lib.mfa_stream_read.restype = ctypes.c_int
    lib.mfa_kv_append.argtypes = [ctypes.POINTER(MfaKvAppendDesc), P, P, P, P, P, P, P, P, P, P]
    lib.mfa_kv_append.restype = ctypes.c_int
    lib.mfa_kv_append_layout.argtypes = [ctypes.POINTER(MfaKvAppendDesc), P, P, P, P, P, P, P, P,
                                         P, ctypes.c_int32, P]
    lib.mfa_kv_append_layout.restype = ctypes.c_int
    lib.mfa_query_proj.argtypes = [qp_p, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.mfa_query_proj.restype = ctypes.c_int
    lib.mfa_query_proj_workspace_size.argtypes = [qp_p]
    lib.mfa_query_proj_workspace_size.restype = ctypes.c_size_t
    sp_p = ctypes.POINTER(MfaSparseDesc)
    lib.mfa_sparse_summarize.argtypes = [sp_p, P, P, P, P, P]
    lib.mfa_sparse_summarize.restype = ctypes.c_int
    lib.mfa_sparse_summarize_new.argtypes = [sp_p, P, P, P, ctypes.c_int32, P, P]
    lib.mfa_sparse_summarize_new.restype = ctypes.c_int
    lib.mfa_sparse_select.argtypes = [sp_p, P, P, P, P, P, P, ctypes.c_void_p, ctypes.c_size_t, P]
    lib.mfa_sparse_select.restype = ctypes.c_int
    lib.mfa_sparse_attention.argtypes = [sp_p, P, P, P, P, P, P, P, P, ctypes.c_float, P,
                                         ctypes.c_size_t, P]
    lib.mfa_sparse_attention.restype = ctypes.c_int
    lib.mfa_sparse_workspace_size.argtypes = [sp_p]
    lib.mfa_sparse_workspace_size.restype = ctypes.c_size_t
    lib.mfa_status_string.argtypes = [ctypes.c_int]
    lib.mfa_status_string.restype = ctypes.c_char_p
    lib.mfa_abi_version.argtypes = []
    lib.mfa_abi_version.restype = ctypes.c_int32
    _LIB = lib
    return lib


def check(status):
    """Raise on a non-zero mfa_status."""
    if status != MFA_OK:
        msg = load().mfa_status_string(status).decode()
        raise RuntimeError(f"{STATUS_NAMES.get(status, status)}: {msg}")
