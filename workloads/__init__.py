"""Seeded synthetic inputs for the attention forward pass and the paged decode.

This module only draws random numbers and lays them out in memory. It holds none
of the attention arithmetic, so both the CPU oracle (through the tests and the
benchmark) and the HIP path consume exactly the same bytes without sharing any
code that computes a result.

Every tensor is produced on the CPU from ``numpy.random.Generator(PCG64(seed))``
so the bytes are identical on every machine. Values are drawn as float32
``standard_normal`` in logical order (Q, then K, then V) and rounded to the
storage dtype with torch's round-to-nearest-even casts.

The workload shapes follow the problem statement of the pages: [B, H, N, D]
tensors with the softmax scale 1/sqrt(D) ("Agent 帮我写 CUDA：一个 Softmax
Attention 算子的开发全记录", section 二 "实验环境", test configuration table),
and the scenario axes (GQA, causal / sliding-window / softcap masks, ragged
batches, split-KV decode over a paged KV cache, fp8 KV) listed in "Ask, Don't
Equip: Question-Driven Coding Agents for Deep Kernel Optimization", section
研究动机.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16

_TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.float8_e4m3fn,
}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _normal(rng: np.random.Generator, shape, mul: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mul != 1.0:
        x *= np.float32(mul)
    return x


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPES[dtype])


@dataclasses.dataclass
class PrefillCase:
    """One prefill problem.

    Dense layout: q [B, Hq, Nq, D], k/v [B, Hkv, Nk, D].
    Ragged (varlen) layout: q [T, Hq, D], k/v [T, Hkv, D] with sequences packed
    token-major and delimited by ``cu_seqlens`` ([B+1] int32, starting at 0).
    """
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    dtype: str
    causal: bool = False
    window: int = 0
    softcap: float = 0.0
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None
    seed: int = 0

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens_q is not None


def make_prefill(*, batch: int, num_q_heads: int, num_kv_heads: int, seqlen_q: int,
                 seqlen_k: Optional[int] = None, head_dim: int, dtype: str, seed,
                 input_scale: float = 1.0, causal: bool = False, window: int = 0,
                 softcap: float = 0.0) -> PrefillCase:
    """Dense [B, H, N, D] inputs, iid N(0,1) times ``input_scale``."""
    seqlen_k = seqlen_q if seqlen_k is None else seqlen_k
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (batch, num_q_heads, seqlen_q, head_dim), input_scale)
    k = _normal(rng, (batch, num_kv_heads, seqlen_k, head_dim), input_scale)
    v = _normal(rng, (batch, num_kv_heads, seqlen_k, head_dim), input_scale)
    return PrefillCase(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), batch=batch,
                       num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, seqlen_q=seqlen_q,
                       seqlen_k=seqlen_k, head_dim=head_dim, dtype=dtype, causal=causal,
                       window=window, softcap=softcap,
                       seed=seed if isinstance(seed, int) else 0)


def make_prefill_varlen(*, lengths_q: Sequence[int], lengths_k: Optional[Sequence[int]] = None,
                        num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str, seed,
                        input_scale: float = 1.0, causal: bool = True, window: int = 0,
                        softcap: float = 0.0) -> PrefillCase:
    """Ragged batch packed token-major: q [T, Hq, D], k/v [Tk, Hkv, D]."""
    lengths_q = [int(x) for x in lengths_q]
    lengths_k = lengths_q if lengths_k is None else [int(x) for x in lengths_k]
    cu_q = np.zeros(len(lengths_q) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(lengths_q)
    cu_k = np.zeros(len(lengths_k) + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(lengths_k)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (int(cu_q[-1]), num_q_heads, head_dim), input_scale)
    k = _normal(rng, (int(cu_k[-1]), num_kv_heads, head_dim), input_scale)
    v = _normal(rng, (int(cu_k[-1]), num_kv_heads, head_dim), input_scale)
    return PrefillCase(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                       batch=len(lengths_q), num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       seqlen_q=max(lengths_q), seqlen_k=max(lengths_k), head_dim=head_dim,
                       dtype=dtype, causal=causal, window=window, softcap=softcap,
                       cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                       seed=seed if isinstance(seed, int) else 0)


@dataclasses.dataclass
class DecodeCase:
    """One paged decode problem.

    q: [S, Hq, D] (bf16/f16). Caches: [num_pages + 1, PAGE_SIZE, Hkv, D] where the
    last page (id ``poison_page``) is NaN-filled and pads every block-table row.
    block_table: [S, max_pages] int32; seq_lens: [S] int32 (includes the current
    token). For fp8 KV the caches hold e4m3fn codes and ``k_scale``/``v_scale``
    ([Hkv] float32) give the per-head dequantisation scale (value = code * scale).
    ``k_logical``/``v_logical`` (optional) are the per-sequence logical tensors
    [L_s, Hkv, D] before paging, kept only when requested (tiny cases).
    """
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: np.ndarray
    seq_lens: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    kv_dtype: str
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    poison_page: int = 0
    k_logical: Optional[list] = None
    v_logical: Optional[list] = None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def make_decode(*, lengths: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                q_dtype: str = "bf16", kv_dtype: str = "bf16", seed: int,
                scale_low: float = 0.5, scale_high: float = 2.0, pow2_scales: bool = False,
                keep_logical: bool = False, max_pages: Optional[int] = None) -> DecodeCase:
    """Paged KV cache with randomly permuted physical pages.

    Draw order: page permutation and (fp8) scales from the root generator, Q,
    then per sequence s the K and V values from child generator s (so the host
    never holds a full float32 copy of the cache).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    S = int(lengths.shape[0])
    D, Hkv, Hq = head_dim, num_kv_heads, num_q_heads
    pages_per_seq = (lengths + PAGE_SIZE - 1) // PAGE_SIZE
    total_pages = int(pages_per_seq.sum())
    max_p = int(pages_per_seq.max()) if max_pages is None else int(max_pages)
    root = np.random.SeedSequence(seed)
    children = root.spawn(S + 1)
    rng = np.random.Generator(np.random.PCG64(children[S]))
    perm = rng.permutation(total_pages).astype(np.int32)
    poison = total_pages
    k_scale = v_scale = None
    if kv_dtype == "fp8_e4m3":
        if pow2_scales:
            k_scale = (2.0 ** rng.integers(-1, 2, size=Hkv)).astype(np.float32)
            v_scale = (2.0 ** rng.integers(-1, 2, size=Hkv)).astype(np.float32)
        else:
            k_scale = rng.uniform(scale_low, scale_high, size=Hkv).astype(np.float32)
            v_scale = rng.uniform(scale_low, scale_high, size=Hkv).astype(np.float32)
    q = _cast(_normal(rng, (S, Hq, D)), q_dtype)

    store = "bf16" if kv_dtype == "bf16" else kv_dtype
    tdt = _TORCH_DTYPES[store]
    k_cache = torch.empty((total_pages + 1, PAGE_SIZE, Hkv, D), dtype=tdt)
    v_cache = torch.empty((total_pages + 1, PAGE_SIZE, Hkv, D), dtype=tdt)
    nan = torch.full((PAGE_SIZE, Hkv, D), float("nan"), dtype=torch.float32).to(tdt)
    k_cache[poison] = nan
    v_cache[poison] = nan
    block_table = np.full((S, max_p), poison, dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(pages_per_seq)]).astype(np.int64)

    def one_sequence(s):
        L = int(lengths[s])
        n_p = int(pages_per_seq[s])
        crng = np.random.Generator(np.random.PCG64(children[s]))
        out = []
        for scale in ((k_scale, v_scale) if kv_dtype == "fp8_e4m3" else (None, None)):
            x = _normal(crng, (L, Hkv, D))
            if scale is not None:
                x /= scale[None, :, None]
            t = torch.empty((n_p * PAGE_SIZE, Hkv, D), dtype=tdt)
            t[:L] = torch.from_numpy(x).to(tdt)
            if n_p * PAGE_SIZE > L:
                t[L:] = nan[0, 0, 0]
            out.append(t.view(n_p, PAGE_SIZE, Hkv, D))
        return out

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    k_log, v_log = ([], []) if keep_logical else (None, None)
    with ThreadPoolExecutor(workers) as ex:
        for s, (kt, vt) in enumerate(ex.map(one_sequence, range(S))):
            n_p = int(pages_per_seq[s])
            ids = perm[offsets[s]:offsets[s] + n_p]
            idx = torch.from_numpy(ids).long()
            k_cache[idx] = kt
            v_cache[idx] = vt
            block_table[s, :n_p] = ids
            if keep_logical:
                L = int(lengths[s])
                k_log.append(kt.reshape(n_p * PAGE_SIZE, Hkv, D)[:L].clone())
                v_log.append(vt.reshape(n_p * PAGE_SIZE, Hkv, D)[:L].clone())
    return DecodeCase(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                      seq_lens=lengths.astype(np.int32), num_q_heads=Hq, num_kv_heads=Hkv,
                      head_dim=D, q_dtype=q_dtype, kv_dtype=kv_dtype, k_scale=k_scale,
                      v_scale=v_scale, poison_page=poison, k_logical=k_log, v_logical=v_log)


@dataclasses.dataclass
class PagedPrefillCase:
    """Chunked prefill over a paged cache: chunk b's queries q[cu_seqlens_q[b]:cu_seqlens_q[b+1]]
    ([T, Hq, D] packed) are the last positions of sequence b, whose seq_lens_k[b] keys (the
    chunk's own included) sit in ``cache``'s pages (``cache.q`` is unused)."""
    q: torch.Tensor
    cu_seqlens_q: np.ndarray
    cache: DecodeCase
    causal: bool = True
    window: int = 0
    softcap: float = 0.0

    @property
    def seq_lens_k(self) -> np.ndarray:
        return self.cache.seq_lens

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if len(self.cu_seqlens_q) > 1 else 0


def make_paged_prefill(*, lengths_q: Sequence[int], lengths_k: Sequence[int], num_q_heads: int,
                       num_kv_heads: int, head_dim: int, dtype: str = "bf16", seed: int,
                       causal: bool = True, window: int = 0, softcap: float = 0.0,
                       keep_logical: bool = False, max_pages: Optional[int] = None) -> PagedPrefillCase:
    """The cache as make_decode draws it (seed), then Q iid N(0,1) from a generator of its
    own (seed + 1_000_003)."""
    lengths_q = [int(x) for x in lengths_q]
    cache = make_decode(lengths=lengths_k, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, q_dtype=dtype, kv_dtype=dtype, seed=seed,
                        keep_logical=keep_logical, max_pages=max_pages)
    cu = np.zeros(len(lengths_q) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths_q)
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    q = _cast(_normal(rng, (int(cu[-1]), num_q_heads, head_dim)), dtype)
    return PagedPrefillCase(q=q, cu_seqlens_q=cu, cache=cache, causal=causal, window=window,
                            softcap=softcap)


# ----------------------------------------------------------------------------------------
# The five workload families of the problem statement, by name.
# ----------------------------------------------------------------------------------------

def config_small_f32(seed: int = 1) -> PrefillCase:
    """Dense non-causal, fp32, B=2 H=4 N=64 D=32 (the page's first correctness shape)."""
    return make_prefill(batch=2, num_q_heads=4, num_kv_heads=4, seqlen_q=64, head_dim=32,
                        dtype="f32", seed=seed)


SWEEP_N = (512, 1024, 2048, 4096)
SWEEP_D = (32, 64, 128)


def config_sweep(n: int, d: int, dtype: str, seed: int = 2) -> PrefillCase:
    """Dense non-causal sweep point, B=2 H=8; one SeedSequence child per (N, D, dtype)."""
    idx = (SWEEP_N.index(n) * len(SWEEP_D) + SWEEP_D.index(d)) * 2 + (0 if dtype == "f32" else 1)
    child = np.random.SeedSequence(seed).spawn(len(SWEEP_N) * len(SWEEP_D) * 2)[idx]
    return make_prefill(batch=2, num_q_heads=8, num_kv_heads=8, seqlen_q=n, head_dim=d,
                        dtype=dtype, seed=child)


def config_headline(seed: int = 3) -> PrefillCase:
    """Full-sequence dense non-causal bf16, B=1 H=32 N=8192 D=128, inputs 0.5*N(0,1)."""
    return make_prefill(batch=1, num_q_heads=32, num_kv_heads=32, seqlen_q=8192, head_dim=128,
                        dtype="bf16", seed=seed, input_scale=0.5)


GQA_VARIANTS = ("causal", "window", "softcap", "ragged")


def config_gqa(variant: str, seed: int = 4, n: int = 4096, batch: int = 4) -> PrefillCase:
    """Causal GQA prefill bf16, B=4 Hq=32 Hkv=8 N=4096 D=128 and its three variants."""
    child = np.random.SeedSequence(seed).spawn(len(GQA_VARIANTS))[GQA_VARIANTS.index(variant)]
    common = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
    if variant == "ragged":
        rng = np.random.Generator(np.random.PCG64(child))
        lengths = rng.integers(n // 4, n, endpoint=True, size=batch)
        sub = np.random.SeedSequence(int(rng.integers(0, 2**63)))
        return make_prefill_varlen(lengths_q=lengths, seed=sub, causal=True, **common)
    window = 1024 if variant == "window" else 0
    softcap = 30.0 if variant == "softcap" else 0.0
    return make_prefill(batch=batch, seqlen_q=n, seed=child, causal=True, window=window,
                        softcap=softcap, **common)


def decode_lengths(seed: int = 5, num_seqs: int = 64, lo: int = 512, hi: int = 32768) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(2)[0]))
    return rng.integers(lo, hi, endpoint=True, size=num_seqs)


def config_decode(kv_dtype: str, seed: int = 5, num_seqs: int = 64,
                  lengths: Optional[Sequence[int]] = None, num_kv_heads: int = 8) -> DecodeCase:
    """Split-KV paged decode: 64 sequences, Hq=32 Hkv=8 D=128, L ~ U[512, 32768]
    (num_kv_heads=1: the MQA form of the same workload)."""
    if lengths is None:
        lengths = decode_lengths(seed, num_seqs)
    child = np.random.SeedSequence(seed).spawn(2)[1]
    sub = int(np.random.Generator(np.random.PCG64(child)).integers(0, 2**63))
    return make_decode(lengths=lengths, num_q_heads=32, num_kv_heads=num_kv_heads, head_dim=128,
                       q_dtype="bf16", kv_dtype=kv_dtype, seed=sub + (1 if kv_dtype != "bf16" else 0))


# ----------------------------------------------------------------------------------------
# Dominance probes: inputs where, for every query, one chosen key scores far above all
# others, so the exact result is that key's value row. Keys carry their position as a
# one-hot digit code; a query carries the code of its target scaled by ``amp``. A key
# matching all digits scores 3*amp, one differing in a digit at most 2*amp.
# ----------------------------------------------------------------------------------------

def chunked_prefill_lengths(seed: int = 6, num_seqs: int = 8, chunk: int = 2048,
                            max_context: int = 14336):
    """A chunk of ``chunk`` new tokens per sequence after a cached context of uniform length
    in [0, max_context]: (lengths_q, lengths_k)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(0, max_context + 1, size=num_seqs)
    return [chunk] * num_seqs, [int(c) + chunk for c in ctx]


def config_chunked_prefill(seed: int = 6, num_seqs: int = 8, chunk: int = 2048,
                           max_context: int = 14336) -> PagedPrefillCase:
    """Chunked prefill after the causal GQA family (Hq=32, Hkv=8, D=128, bf16, values
    N(0,1)): chunks of 2048 queries over contexts uniform in [0, 14336] in 16-token pages
    at randomly permuted block-table indices."""
    lq, lk = chunked_prefill_lengths(seed, num_seqs, chunk, max_context)
    return make_paged_prefill(lengths_q=lq, lengths_k=lk, num_q_heads=32, num_kv_heads=8,
                              head_dim=128, dtype="bf16", seed=seed)


@dataclasses.dataclass
class Fp8PrefillCase:
    """Dense prefill on fp8 e4m3 codes [B, H, N, D] (torch.float8_e4m3fn) with per-tensor
    scales (value = code * scale); the output is bf16."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_scale: float
    k_scale: float
    v_scale: float
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    causal: bool = False
    window: int = 0
    softcap: float = 0.0


def make_prefill_fp8(*, batch: int, num_q_heads: int, num_kv_heads: int, seqlen_q: int,
                     seqlen_k: Optional[int] = None, head_dim: int, seed, input_scale: float = 1.0,
                     causal: bool = False, window: int = 0, softcap: float = 0.0) -> Fp8PrefillCase:
    """Q, K, V drawn as make_prefill draws them, then stored as e4m3 codes of x / s with
    one scale per tensor, s = max|x| / 448 (the codes span the format's range)."""
    seqlen_k = seqlen_q if seqlen_k is None else seqlen_k
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for shape in ((batch, num_q_heads, seqlen_q, head_dim), (batch, num_kv_heads, seqlen_k, head_dim),
                  (batch, num_kv_heads, seqlen_k, head_dim)):
        x = _normal(rng, shape, input_scale)
        sc = np.float32(max(float(np.abs(x).max()), 1e-30) / 448.0)
        out.append((_cast(x / sc, "fp8_e4m3"), float(sc)))
    (q, qs), (k, ks), (v, vs) = out
    return Fp8PrefillCase(q=q, k=k, v=v, q_scale=qs, k_scale=ks, v_scale=vs, batch=batch,
                          num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, seqlen_q=seqlen_q,
                          seqlen_k=seqlen_k, head_dim=head_dim, causal=causal, window=window,
                          softcap=softcap)


def config_fp8_headline(seed: int = 9) -> Fp8PrefillCase:
    """The headline shape (B=1 H=32 N=8192 D=128, dense, inputs 0.5 N(0,1)) on fp8 e4m3
    inputs with per-tensor scales."""
    return make_prefill_fp8(batch=1, num_q_heads=32, num_kv_heads=32, seqlen_q=8192, head_dim=128,
                            seed=seed, input_scale=0.5)


def make_grad_out(shape, *, dtype: str = "bf16", seed: int) -> torch.Tensor:
    """dL/dO for the backward: iid N(0,1) in ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _cast(_normal(rng, tuple(shape)), dtype)


def config_backward(seed: int = 10) -> PrefillCase:
    """Causal GQA bf16 prefill for the backward: B=1 Hq=32 Hkv=8 N=4096 D=128, inputs
    N(0,1) (dL/dO from make_grad_out with seed + 1)."""
    return make_prefill(batch=1, num_q_heads=32, num_kv_heads=8, seqlen_q=4096, head_dim=128, dtype="bf16",
                        seed=seed, causal=True)


def config_headdim(head_dim: int, seed: int = 8) -> PrefillCase:
    """Causal prefill bf16 B=2 H=16 N=4096 at the head dims without a dedicated workload
    (96, 192, 256); Q, K, V iid N(0,1)."""
    return make_prefill(batch=2, num_q_heads=16, num_kv_heads=16, seqlen_q=4096, head_dim=head_dim,
                        dtype="bf16", seed=seed + head_dim, causal=True)


def position_code(pos: np.ndarray, dim: int, base: int = 16, digits: int = 3) -> np.ndarray:
    """[len(pos), dim] float32 one-hot digit code of each position (base ** digits > pos)."""
    pos = np.asarray(pos, dtype=np.int64)
    if base * digits > dim:
        raise ValueError("code does not fit the head dimension")
    out = np.zeros((pos.shape[0], dim), dtype=np.float32)
    rest = pos.copy()
    for dgt in range(digits):
        out[np.arange(pos.shape[0]), dgt * base + rest % base] = 1.0
        rest //= base
    if (rest != 0).any():
        raise ValueError("position exceeds the code range")
    return out


def dominance_prefill(*, batch: int, num_q_heads: int, num_kv_heads: int, seqlen: int, head_dim: int,
                      dtype: str, targets: np.ndarray, seed: int, amp: float = 512.0,
                      causal: bool = False, window: int = 0, base: int = 16) -> PrefillCase:
    """Dense self-attention probe: query i of every (b, h) targets key targets[i]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    digits = int(np.ceil(np.log(max(seqlen, 2)) / np.log(base)))
    kcode = position_code(np.arange(seqlen), head_dim, base, digits)
    qcode = position_code(np.asarray(targets), head_dim, base, digits) * np.float32(amp)
    q = np.broadcast_to(qcode, (batch, num_q_heads, seqlen, head_dim)).copy()
    k = np.broadcast_to(kcode, (batch, num_kv_heads, seqlen, head_dim)).copy()
    v = _normal(rng, (batch, num_kv_heads, seqlen, head_dim))
    return PrefillCase(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), batch=batch,
                       num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, seqlen_q=seqlen,
                       seqlen_k=seqlen, head_dim=head_dim, dtype=dtype, causal=causal, window=window,
                       seed=seed)


def dominance_decode(case: DecodeCase, targets: np.ndarray, amp: float = 1024.0,
                     base: int = 32) -> DecodeCase:
    """Overwrite a decode case's K cache and Q with the digit code: query (s, h) targets
    logical token targets[s, h] of sequence s. For fp8 caches the stored K code is
    1/k_scale times the digit (choose power-of-two scales so it is exact)."""
    S, Hq, D = case.q.shape
    Hkv = case.num_kv_heads
    digits = 3
    kc = torch.zeros_like(case.k_cache, dtype=torch.float32)
    kc[case.poison_page] = float("nan")
    for s in range(S):
        L = int(case.seq_lens[s])
        t = np.arange(L)
        code = torch.from_numpy(position_code(t, D, base, digits))  # [L, D]
        phys = torch.from_numpy(case.block_table[s, t // PAGE_SIZE].astype(np.int64))
        slot = torch.from_numpy((t % PAGE_SIZE).astype(np.int64))
        vals = code[:, None, :].expand(L, Hkv, D)
        if case.k_scale is not None:
            vals = vals / torch.from_numpy(case.k_scale)[None, :, None]
        kc[phys, slot] = vals
        tail = torch.arange(L, ((L + PAGE_SIZE - 1) // PAGE_SIZE) * PAGE_SIZE)
        if tail.numel():
            kc[torch.from_numpy(case.block_table[s, tail.numpy() // PAGE_SIZE].astype(np.int64)),
               tail % PAGE_SIZE] = float("nan")
    qv = position_code(np.asarray(targets).reshape(-1), D, base, digits).reshape(S, Hq, D) * np.float32(amp)
    return dataclasses.replace(case, k_cache=kc.to(case.k_cache.dtype), q=_cast(qv, case.q_dtype))
