"""MI355X (gfx950) fused attention forward: Python binding of libattn.so.

Every step of the computation runs in the HIP kernels behind the C ABI of
include/attn.h; this module only checks tensor metadata, allocates outputs
with torch (device memory and the current stream are torch's), and passes
pointers. If the library is missing it raises: there is no CPU fallback.

    fwd(q, k, v, ...)            softmax(Q K^T * scale [+ mask]) V (prefill)
    fwd_paged(q, k_cache, ...)    chunked prefill over a paged cache
    bwd(q, k, v, o, dout, lse)    gradients of fwd (dense batches)
    decode_paged(q, k_cache, ...) one query token per sequence over a paged cache
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import AttnError, AttnInvalidValue, AttnNotSupported

__all__ = ["fwd", "fwd_paged", "bwd", "bwd_workspace_size", "fwd_paged_workspace_size", "decode_paged", "decode_paged_noalloc", "decode_plan", "decode_workspace_size", "library_path",
           "AttnError", "AttnInvalidValue", "AttnNotSupported"]

_DTYPES = {torch.float32: _lib.ATTN_F32, torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16,
           torch.float8_e4m3fn: _lib.ATTN_FP8_E4M3}


def library_path() -> str:
    _lib.lib()
    return _lib.LIB_PATH


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _sinks_ptr(sinks: Optional[torch.Tensor], hq: int) -> Optional[int]:
    if sinks is None:
        return None
    if sinks.dtype != torch.float32 or not sinks.is_contiguous() or sinks.shape != (hq,) or not sinks.is_cuda:
        raise ValueError(f"sinks must be a contiguous float32 GPU tensor of shape ({hq},)")
    return sinks.data_ptr()


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False, window: int = 0,
        softcap: float = 0.0, softmax_scale: float = 0.0, cu_seqlens_q: Optional[torch.Tensor] = None,
        cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
        max_seqlen_k: Optional[int] = None, return_lse: bool = False, out: Optional[torch.Tensor] = None,
        lse_out: Optional[torch.Tensor] = None, sinks: Optional[torch.Tensor] = None,
        q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0):
    """Fused attention forward.

    Dense: q [B, Hq, Nq, D], k/v [B, Hkv, Nk, D] (any strides with D contiguous).
    Ragged: q [T, Hq, D], k/v [Tk, Hkv, D] with int32 cu_seqlens_q/k [B+1] on the
    GPU and host-side upper bounds max_seqlen_q/k.
    Returns o (like q), and lse (float32; dense [B, Hq, Nq], ragged [Hq, T]) if
    return_lse. sinks: optional float32 [Hq] per-head sink logits (natural log).
    float8_e4m3fn q/k/v (head_dim 128) take per-tensor scales q_scale / k_scale /
    v_scale (value = code * scale) and give a bfloat16 o.
    """
    _require_cuda(q, k, v, sinks)
    if q.dtype not in (torch.float32, torch.float16, torch.bfloat16, torch.float8_e4m3fn):
        raise AttnNotSupported(_lib.ATTN_ERROR_NOT_SUPPORTED, f"dtype {q.dtype} not supported")
    out_dtype = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share a dtype")
    ragged = cu_seqlens_q is not None
    a = _lib.FwdArgs()
    if ragged:
        if cu_seqlens_k is None or max_seqlen_q is None or max_seqlen_k is None:
            raise ValueError("ragged batches need cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k")
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("ragged q/k/v must be [T, H, D]")
        for cu in (cu_seqlens_q, cu_seqlens_k):
            if cu.dtype != torch.int32 or not cu.is_cuda or cu.dim() != 1 or not cu.is_contiguous():
                raise ValueError("cu_seqlens must be contiguous int32 GPU vectors")
        a.batch = cu_seqlens_q.numel() - 1
        a.num_q_heads, a.num_kv_heads, a.head_dim = q.shape[1], k.shape[1], q.shape[2]
        a.seqlen_q, a.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        qs = (0, q.stride(1), q.stride(0))
        ks = (0, k.stride(1), k.stride(0))
        vs = (0, v.stride(1), v.stride(0))
        a.cu_seqlens_q = cu_seqlens_q.data_ptr()
        a.cu_seqlens_k = cu_seqlens_k.data_ptr()
        lse_shape = (q.shape[1], q.shape[0])
    else:
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("dense q/k/v must be [B, H, N, D]")
        a.batch, a.num_q_heads, a.seqlen_q, a.head_dim = q.shape
        a.num_kv_heads, a.seqlen_k = k.shape[1], k.shape[2]
        if k.shape[0] != q.shape[0] or v.shape[:3] != k.shape[:3]:
            raise ValueError("k/v shapes do not match q")
        qs = (q.stride(0), q.stride(1), q.stride(2))
        ks = (k.stride(0), k.stride(1), k.stride(2))
        vs = (v.stride(0), v.stride(1), v.stride(2))
        lse_shape = (q.shape[0], q.shape[1], q.shape[2])
    if q.stride(-1) != 1 or k.stride(-1) != 1 or v.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    if k.shape[-1] != a.head_dim or v.shape[-1] != a.head_dim:
        raise ValueError("q, k and v must share head_dim")
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device) if out is None else out
    if o.shape != q.shape or o.dtype != out_dtype or o.stride(-1) != 1:
        raise ValueError(f"out must have q's shape and dtype {out_dtype}")
    os_ = (0, o.stride(1), o.stride(0)) if ragged else (o.stride(0), o.stride(1), o.stride(2))
    lse = None
    if return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device) if lse_out is None else lse_out
        if lse.shape != lse_shape or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse_out must be a contiguous float32 tensor of shape {lse_shape}")
    a.dtype = _DTYPES[q.dtype]
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.softmax_scale = float(softmax_scale)
    a.softcap = float(softcap)
    a.sinks = _sinks_ptr(sinks, a.num_q_heads)
    a.q_scale, a.k_scale, a.v_scale = float(q_scale), float(k_scale), float(v_scale)
    for name, st in (("q_stride", qs), ("k_stride", ks), ("v_stride", vs), ("o_stride", os_)):
        arr = getattr(a, name)
        for i in range(3):
            arr[i] = int(st[i])
    status = _lib.lib().attn_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 _stream_handle(q.device))
    _lib.check(status)
    return (o, lse) if return_lse else o


def fwd_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
              cu_seqlens_q: torch.Tensor, seq_lens_k: torch.Tensor, max_seqlen_q: int, *, causal: bool = True,
              window: int = 0, softcap: float = 0.0, softmax_scale: float = 0.0, return_lse: bool = False,
              out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, gather: bool = True,
              sinks: Optional[torch.Tensor] = None):
    """Chunked prefill over a paged KV cache.

    q [T, Hq, D] packed chunks (int32 cu_seqlens_q [S+1] on the GPU, max_seqlen_q a
    host-side bound of the chunk lengths); k_cache/v_cache [P, 16, Hkv, D] in q's
    dtype (bf16/f16); block_table int32 [S, max_pages]; seq_lens_k int32 [S], the
    keys of each sequence, the chunk's own included. Returns o [T, Hq, D] (and lse
    [Hq, T] float32 if return_lse).

    gather: use the gathered-key route where the library has one (a workspace of
    fwd_paged_workspace_size bytes, allocated here unless ``workspace`` is given);
    gather=False reads the pages in place.
    """
    _require_cuda(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k, sinks)
    for t in (q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k):
        if not t.is_contiguous():
            raise ValueError("paged prefill tensors must be contiguous")
    if block_table.dtype != torch.int32 or cu_seqlens_q.dtype != torch.int32 or seq_lens_k.dtype != torch.int32:
        raise ValueError("block_table, cu_seqlens_q and seq_lens_k must be int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must match each other and q's dtype")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape[3] != q.shape[2]:
        raise ValueError("q must be [T, Hq, D] and the caches [P, page, Hkv, D]")
    S = seq_lens_k.numel()
    if block_table.dim() != 2 or block_table.shape[0] != S or cu_seqlens_q.shape != (S + 1,):
        raise ValueError("block_table must be [S, max_pages] and cu_seqlens_q [S + 1]")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise AttnNotSupported(_lib.ATTN_ERROR_NOT_SUPPORTED, f"dtype {q.dtype} not supported")
    a = _lib.FwdPagedArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = S, q.shape[1], k_cache.shape[2], q.shape[2]
    a.page_size, a.max_pages_per_seq, a.num_pages = k_cache.shape[1], block_table.shape[1], k_cache.shape[0]
    a.max_seqlen_q = int(max_seqlen_q)
    a.dtype = _DTYPES[q.dtype]
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.softmax_scale = float(softmax_scale)
    a.softcap = float(softcap)
    a.sinks = _sinks_ptr(sinks, a.num_q_heads)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must match q")
    lse = None
    if return_lse:
        shape = (q.shape[1], q.shape[0])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device) if lse_out is None else lse_out
        if lse.shape != shape or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse_out must be a contiguous float32 tensor of shape {shape}")
    L = _lib.lib()
    ws_bytes = 0
    if gather:
        need = int(L.attn_fwd_paged_workspace_size(ctypes.byref(a)))
        if need > 0 and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if need == 0:
            workspace = None
    else:
        workspace = None
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not workspace.is_cuda:
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        ws_bytes = workspace.numel()
    status = L.attn_fwd_paged(ctypes.byref(a), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                              _ptr(cu_seqlens_q), _ptr(seq_lens_k), _ptr(o), _ptr(lse), _ptr(workspace),
                              ws_bytes, _stream_handle(q.device))
    _lib.check(status)
    return (o, lse) if return_lse else o


def fwd_paged_workspace_size(*, num_seqs, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, num_pages,
                             dtype, max_seqlen_q=1, page_size=16) -> int:
    """Bytes of workspace the gathered route of fwd_paged uses (0: no such route)."""
    a = _lib.FwdPagedArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = num_seqs, num_q_heads, num_kv_heads, head_dim
    a.page_size, a.max_pages_per_seq, a.num_pages, a.max_seqlen_q = page_size, max_pages_per_seq, num_pages, max_seqlen_q
    a.dtype = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    a.causal = 1
    return int(_lib.lib().attn_fwd_paged_workspace_size(ctypes.byref(a)))


def bwd_workspace_size(q: torch.Tensor, k: torch.Tensor, *, causal: bool = False, window: int = 0) -> int:
    """Bytes of workspace bwd needs for q [B, Hq, Nq, D] and k [B, Hkv, Nk, D]."""
    a = _lib.BwdArgs()
    a.batch, a.num_q_heads, a.seqlen_q, a.head_dim = q.shape
    a.num_kv_heads, a.seqlen_k = k.shape[1], k.shape[2]
    a.dtype = _DTYPES[q.dtype]
    a.causal = 1 if causal else 0
    a.window = int(window)
    return int(_lib.lib().attn_bwd_workspace_size(ctypes.byref(a)))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
        lse: torch.Tensor, *, causal: bool = False, window: int = 0, softcap: float = 0.0,
        softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None,
        dq_out: Optional[torch.Tensor] = None, dk_out: Optional[torch.Tensor] = None,
        dv_out: Optional[torch.Tensor] = None):
    """Gradients of fwd for dense batches: q, o, dout [B, Hq, Nq, D]; k, v [B, Hkv, Nk, D]
    (contiguous, bf16/f16); lse float32 [B, Hq, Nq] from fwd(..., return_lse=True).
    Returns (dq, dk, dv), written into dq_out / dk_out / dv_out when given (contiguous,
    shapes and dtype of q, k, v)."""
    _require_cuda(q, k, v, o, dout, lse)
    for t in (q, k, v, o, dout, lse):
        if not t.is_contiguous():
            raise ValueError("backward tensors must be contiguous")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise AttnNotSupported(_lib.ATTN_ERROR_NOT_SUPPORTED, f"dtype {q.dtype} not supported")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)) or lse.dtype != torch.float32:
        raise ValueError("q, k, v, o, dout share a 16-bit dtype; lse is float32")
    if q.dim() != 4 or k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B, Hq, Nq, D] and k, v [B, Hkv, Nk, D]")
    if lse.shape != q.shape[:3]:
        raise ValueError("lse must be [B, Hq, Nq]")
    a = _lib.BwdArgs()
    a.batch, a.num_q_heads, a.seqlen_q, a.head_dim = q.shape
    a.num_kv_heads, a.seqlen_k = k.shape[1], k.shape[2]
    a.dtype = _DTYPES[q.dtype]
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.softmax_scale = float(softmax_scale)
    a.softcap = float(softcap)
    L = _lib.lib()
    need = int(L.attn_bwd_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    grads = []
    for given, like, name in ((dq_out, q, "dq_out"), (dk_out, k, "dk_out"), (dv_out, v, "dv_out")):
        g = torch.empty_like(like) if given is None else given
        if g.shape != like.shape or g.dtype != like.dtype or not g.is_contiguous() or g.device != like.device:
            raise ValueError(f"{name} must be contiguous with the shape and dtype of its input")
        grads.append(g)
    dq, dk, dv = grads
    status = L.attn_bwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                        _stream_handle(q.device))
    _lib.check(status)
    return dq, dk, dv


def _decode_args(*, num_seqs, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq, max_seq_len,
                 q_dtype, kv_dtype, softmax_scale=0.0, num_splits=0, page_size=16, sinks=None) -> _lib.DecodeArgs:
    a = _lib.DecodeArgs()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = num_seqs, num_q_heads, num_kv_heads, head_dim
    a.page_size = page_size
    a.max_pages_per_seq = max_pages_per_seq
    a.max_seq_len = int(max_seq_len)
    a.q_dtype = _DTYPES[q_dtype] if isinstance(q_dtype, torch.dtype) else int(q_dtype)
    a.kv_dtype = _DTYPES[kv_dtype] if isinstance(kv_dtype, torch.dtype) else int(kv_dtype)
    a.softmax_scale = float(softmax_scale)
    a.num_splits = int(num_splits)
    a.sinks = sinks
    return a


def decode_plan(**kw):
    """(split_len, max_splits) the library uses for these decode arguments."""
    a = _decode_args(**kw)
    n_len, n_max = ctypes.c_int32(), ctypes.c_int32()
    _lib.check(_lib.lib().attn_decode_plan(ctypes.byref(a), ctypes.byref(n_len), ctypes.byref(n_max)))
    return n_len.value, n_max.value


def decode_workspace_size(**kw) -> int:
    a = _decode_args(**kw)
    return int(_lib.lib().attn_decode_paged_workspace_size(ctypes.byref(a)))


def decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, max_seq_len: int, *, k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None, softmax_scale: float = 0.0, num_splits: int = 0,
                 return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                 sinks: Optional[torch.Tensor] = None):
    """Paged split-KV decode.

    q [S, Hq, D]; k_cache/v_cache [P, 16, Hkv, D] (bf16/f16, or float8_e4m3fn with
    float32 k_scale/v_scale [Hkv]); block_table int32 [S, max_pages]; seq_lens int32
    [S]; max_seq_len a host-side bound of seq_lens. Returns o [S, Hq, D] (and lse
    [S, Hq] float32 if return_lse), written into out / lse_out when given.
    """
    _require_cuda(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks)
    for t in (q, k_cache, v_cache, block_table, seq_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must be [P, page, Hkv, D] of one dtype")
    S, hq, d = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_table must be [S, max_pages] and seq_lens [S]")
    kw = dict(num_seqs=S, num_q_heads=hq, num_kv_heads=k_cache.shape[2], head_dim=d,
              max_pages_per_seq=block_table.shape[1], max_seq_len=max_seq_len, q_dtype=q.dtype,
              kv_dtype=k_cache.dtype, softmax_scale=softmax_scale, num_splits=num_splits,
              page_size=k_cache.shape[1])
    if k_cache.shape[3] != d:
        raise ValueError("head_dim mismatch between q and the caches")
    for sc in (k_scale, v_scale):
        if sc is not None and (sc.dtype != torch.float32 or not sc.is_contiguous()):
            raise ValueError("k_scale / v_scale must be contiguous float32")
    a = _decode_args(**kw, sinks=_sinks_ptr(sinks, hq))
    L = _lib.lib()
    need = int(L.attn_decode_paged_workspace_size(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must match q")
    lse = None
    if return_lse:
        lse = torch.empty((S, hq), dtype=torch.float32, device=q.device) if lse_out is None else lse_out
        if lse.shape != (S, hq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse_out must be a contiguous float32 tensor of shape ({S}, {hq})")
    status = L.attn_decode_paged(ctypes.byref(a), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                 _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream_handle(q.device))
    _lib.check(status)
    return (o, lse) if return_lse else o


DECODE_NOALLOC_MAX_WORKSPACE = 64 << 20  # bytes: ATTN_DECODE_NOALLOC_MAX_WORKSPACE of include/attn.h


def decode_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, *, out: torch.Tensor, lse_out: Optional[torch.Tensor] = None,
                         k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                         softmax_scale: float = 0.0, num_splits: int = 0, sinks: Optional[torch.Tensor] = None):
    """decode_paged through attn_decode_paged_noalloc: no workspace, and the caller passes the
    outputs (out [S, Hq, D] in q's dtype, optional lse_out float32 [S, Hq]), so the call
    allocates nothing. The per-split partials go to the library's own per-GPU scratch array
    (at most DECODE_NOALLOC_MAX_WORKSPACE bytes; calls that overlap on one GPU race)."""
    _require_cuda(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, out, lse_out)
    for t in (q, k_cache, v_cache, block_table, seq_lens, out):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must be [P, page, Hkv, D] of one dtype")
    S, hq, d = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_table must be [S, max_pages] and seq_lens [S]")
    if k_cache.shape[3] != d:
        raise ValueError("head_dim mismatch between q and the caches")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if lse_out is not None and (lse_out.shape != (S, hq) or lse_out.dtype != torch.float32
                                or not lse_out.is_contiguous()):
        raise ValueError(f"lse_out must be a contiguous float32 tensor of shape ({S}, {hq})")
    for sc in (k_scale, v_scale):
        if sc is not None and (sc.dtype != torch.float32 or not sc.is_contiguous()):
            raise ValueError("k_scale / v_scale must be contiguous float32")
    a = _decode_args(num_seqs=S, num_q_heads=hq, num_kv_heads=k_cache.shape[2], head_dim=d,
                     max_pages_per_seq=block_table.shape[1], max_seq_len=max_seq_len, q_dtype=q.dtype,
                     kv_dtype=k_cache.dtype, softmax_scale=softmax_scale, num_splits=num_splits,
                     page_size=k_cache.shape[1], sinks=_sinks_ptr(sinks, hq))
    status = _lib.lib().attn_decode_paged_noalloc(ctypes.byref(a), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
                                                  _ptr(out), _ptr(lse_out), _stream_handle(q.device))
    _lib.check(status)
    return (out, lse_out) if lse_out is not None else out


# ----------------------------------------------------------------- measurement ----
def probe_mfma(operands: torch.Tensor, clocks: torch.Tensor, sink: torch.Tensor, *, workgroups: int, iters: int,
               valu_mix: bool = False) -> None:
    """Enqueue the matrix-core probe (attn_probe_mfma): operands uint32 [256*8] (as int32),
    clocks int64 [2*workgroups], sink float32 [256*workgroups], all on one GPU."""
    _require_cuda(operands, clocks, sink)
    if operands.numel() < 256 * 8 or clocks.numel() < 2 * workgroups or sink.numel() < 256 * workgroups:
        raise ValueError("probe_mfma: buffers too small")
    L = _lib.lib()
    _lib.check(L.attn_probe_mfma(_ptr(operands), workgroups, iters, 1 if valu_mix else 0, _ptr(clocks), _ptr(sink),
                                 _stream_handle(operands.device)))


def probe_hbm_read(buf: torch.Tensor, sink: torch.Tensor, *, workgroups: int) -> None:
    """Enqueue the streaming-read probe (attn_probe_hbm_read) over all of buf's bytes."""
    _require_cuda(buf, sink)
    if sink.numel() < workgroups:
        raise ValueError("probe_hbm_read: sink too small")
    L = _lib.lib()
    _lib.check(L.attn_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), workgroups, _ptr(sink),
                                     _stream_handle(buf.device)))


def flush_caches(buf: torch.Tensor) -> None:
    """Enqueue a write of zeros over all of buf (attn_flush_caches)."""
    _require_cuda(buf)
    L = _lib.lib()
    _lib.check(L.attn_flush_caches(_ptr(buf), buf.numel() * buf.element_size(), _stream_handle(buf.device)))

