"""ctypes view of the C ABI declared in include/attn.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_SUCCESS = 0
ATTN_ERROR_INVALID_VALUE = 1
ATTN_ERROR_NOT_SUPPORTED = 2
ATTN_ERROR_WORKSPACE_TOO_SMALL = 3
ATTN_ERROR_LAUNCH_FAILED = 4

ATTN_F32 = 0
ATTN_F16 = 1
ATTN_BF16 = 2
ATTN_FP8_E4M3 = 3

EXPORTED = ("attn_fwd", "attn_fwd_paged", "attn_fwd_paged_workspace_size", "attn_bwd", "attn_bwd_workspace_size",
            "attn_decode_plan", "attn_decode_paged_workspace_size", "attn_decode_paged",
            "attn_decode_paged_noalloc",
            "attn_probe_mfma", "attn_probe_hbm_read", "attn_flush_caches",
            "attn_status_string", "attn_last_error_message", "attn_abi_version")


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("sinks", ctypes.c_void_p),
        ("q_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("sinks", ctypes.c_void_p),
    ]


class FwdPagedArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("sinks", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
    ]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libattn.so (built in place); raise if it is missing. There is no fallback."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_forward_03_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_fwd_paged.argtypes = [ctypes.POINTER(FwdPagedArgs)] + [ctypes.c_void_p] * 9 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    L.attn_fwd_paged.restype = ctypes.c_int
    L.attn_fwd_paged_workspace_size.argtypes = [ctypes.POINTER(FwdPagedArgs)]
    L.attn_fwd_paged_workspace_size.restype = ctypes.c_size_t
    L.attn_bwd.argtypes = [ctypes.POINTER(BwdArgs)] + [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p]
    L.attn_bwd.restype = ctypes.c_int
    L.attn_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
    L.attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.attn_decode_plan.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32)]
    L.attn_decode_plan.restype = ctypes.c_int
    L.attn_decode_paged_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs)]
    L.attn_decode_paged_workspace_size.restype = ctypes.c_size_t
    L.attn_decode_paged.argtypes = [ctypes.POINTER(DecodeArgs)] + [ctypes.c_void_p] * 9 + \
        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.attn_decode_paged.restype = ctypes.c_int
    L.attn_decode_paged_noalloc.argtypes = [ctypes.POINTER(DecodeArgs)] + [ctypes.c_void_p] * 10
    L.attn_decode_paged_noalloc.restype = ctypes.c_int
    L.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.attn_probe_mfma.restype = ctypes.c_int
    L.attn_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.attn_probe_hbm_read.restype = ctypes.c_int
    L.attn_flush_caches.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.attn_flush_caches.restype = ctypes.c_int
    L.attn_status_string.argtypes = [ctypes.c_int]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error_message.argtypes = []
    L.attn_last_error_message.restype = ctypes.c_char_p
    L.attn_abi_version.argtypes = []
    L.attn_abi_version.restype = ctypes.c_int32
    _LIB = L
    return L


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class AttnInvalidValue(AttnError, ValueError):
    pass


class AttnNotSupported(AttnError, NotImplementedError):
    pass


def check(status: int) -> None:
    if status == ATTN_SUCCESS:
        return
    L = lib()
    msg = f"{L.attn_status_string(status).decode()}: {L.attn_last_error_message().decode()}"
    if status == ATTN_ERROR_INVALID_VALUE:
        raise AttnInvalidValue(status, msg)
    if status == ATTN_ERROR_NOT_SUPPORTED:
        raise AttnNotSupported(status, msg)
    raise AttnError(status, msg)
