"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same inputs, compare to the stated tolerances.

Tolerances (elementwise, on O and on LSE):
  fp32 inputs          |gpu - oracle| <= 1e-4
  bf16 / f16 inputs    |gpu - oracle| <= 2e-2 + 2e-2 * |oracle|
  fp8 (e4m3) KV, and fp8 Q/K/V prefill
                       |gpu - oracle| <= 6e-2
Because those bounds are loose next to the size of O on nearly-uniform attention,
every comparison also bounds the relative Frobenius error ||gpu - oracle|| / ||oracle||
of O: 1e-5 for fp32 (rounding of fp32 accumulation), 1e-2 for 16-bit inputs (P and O
are rounded to 8 / 11 significant bits: about 2^-9 relative per element), 2e-2 for
fp8 KV (the same, plus the bf16 rounding of Q), 6e-2 for the fp8 prefill (P in e4m3).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {
    "f32": dict(atol=1e-4, rtol=0.0, fro=1e-5),
    "bf16": dict(atol=2e-2, rtol=2e-2, fro=1e-2),
    "f16": dict(atol=2e-2, rtol=2e-2, fro=1e-2),
    "fp8_e4m3": dict(atol=6e-2, rtol=0.0, fro=2e-2),
    # fp8 Q/K/V prefill: P itself is rounded to e4m3 (3 mantissa bits, relative error up to
    # 2^-4, about 3.6% RMS) before the P.V product, so on near-uniform attention O carries
    # that relative error. Per element the error is at most 2^-3 / (1 - 2^-4) times
    # sum_j w_j |v_j - O| plus the bf16 rounding of O; the fp8 prefill tests check that
    # derived bound element by element (tests/test_gpu_fp8_prefill.py) and use this entry
    # for the outer bound (2^-3 times the largest |v| of the test inputs, 13.5) and the
    # Frobenius bound.
    "fp8_prefill": dict(atol=1.7, rtol=0.0, fro=6e-2),
    # gradients (16-bit inputs): sums whose terms can cancel, so the element check is the
    # term-magnitude bound of tests/test_gpu_backward.py; this entry is the outer element
    # bound and the Frobenius bound (the 16-bit one)
    "grad": dict(atol=0.5, rtol=0.02, fro=1e-2),
}


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def widen(t: torch.Tensor, dtype: str) -> np.ndarray:
    return oracle.tensor_to_f64(t.detach().cpu(), dtype)


def compare(got: np.ndarray, ref: np.ndarray, kind: str, what: str, lse: bool = False) -> dict:
    """Assert the tolerance of ``kind``; return error statistics."""
    tol = TOL[kind]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    ninf_ref = np.isneginf(ref)
    assert (np.isneginf(got) == ninf_ref).all(), f"{what}: -inf pattern differs"
    fin = ~ninf_ref
    g, r = got[fin], ref[fin]
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err = np.abs(g - r)
    bound = tol["atol"] + tol["rtol"] * np.abs(r)
    worst = int(np.argmax(err - bound)) if err.size else 0
    assert (err <= bound).all(), (f"{what}: max excess {float((err - bound).max()):.3e} at flat index "
                                  f"{worst} (got {g[worst]!r}, oracle {r[worst]!r})")
    stats = {"max_abs": float(err.max()) if err.size else 0.0}
    if not lse and err.size:
        nr = float(np.linalg.norm(r))
        fro = float(np.linalg.norm(g - r)) / nr if nr > 0 else float(np.linalg.norm(g))
        stats["rel_fro"] = fro
        assert fro <= tol["fro"], f"{what}: relative Frobenius error {fro:.3e} > {tol['fro']}"
    return stats


# ------------------------------------------------------------------- poisoned outputs ----

GUARD = 4096  # elements of NaN on each side of an output buffer


class Guarded:
    """An output tensor that starts as NaN, with NaN guard bands of GUARD elements on both
    sides in the same allocation: an entry the kernels leave unwritten stays NaN (and fails
    the comparison), and a write past either end changes a guard."""

    def __init__(self, shape, dtype, device="cuda"):
        n = int(np.prod(shape))
        self.n = n
        self.buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device=device)
        self.t = self.buf[GUARD:GUARD + n].view(shape)

    def check_guards(self, what: str) -> None:
        b = self.buf.detach().cpu().float()
        lo, hi = b[:GUARD], b[GUARD + self.n:]
        assert bool(torch.isnan(lo).all()) and bool(torch.isnan(hi).all()), f"{what}: a guard band was written"


# ---------------------------------------------------------------------------- prefill ----

def _dev_sinks(sinks):
    return None if sinks is None else torch.as_tensor(np.asarray(sinks, dtype=np.float32)).cuda()


def run_prefill(case, *, return_lse=True, out=None, sinks=None):
    import attention_forward_03_amd as attn
    q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
    kw = dict(causal=case.causal, window=case.window, softcap=case.softcap, return_lse=return_lse,
              sinks=_dev_sinks(sinks))
    if case.varlen:
        kw.update(cu_seqlens_q=torch.from_numpy(case.cu_seqlens_q).cuda(),
                  cu_seqlens_k=torch.from_numpy(case.cu_seqlens_k).cuda(),
                  max_seqlen_q=case.seqlen_q, max_seqlen_k=case.seqlen_k)
    # the outputs start as NaN: an entry the kernels leave unwritten fails the comparison
    kw["out"] = torch.full(q.shape, float("nan"), dtype=q.dtype, device=q.device) if out is None else out
    if return_lse:
        lse_shape = (q.shape[1], q.shape[0]) if case.varlen else tuple(q.shape[:3])
        kw["lse_out"] = torch.full(lse_shape, float("nan"), dtype=torch.float32, device=q.device)
    res = attn.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    if return_lse:
        o, lse = res
        return o.cpu(), lse.cpu()
    return res.cpu(), None


def oracle_prefill(case, *, rows=None, heads=None, seqs=None, sinks=None):
    """Oracle O/LSE for the case (a sample of rows / heads when given), float64."""
    q = oracle.tensor_to_f64(case.q, case.dtype)
    k = oracle.tensor_to_f64(case.k, case.dtype)
    v = oracle.tensor_to_f64(case.v, case.dtype)
    scale = oracle.default_scale(case.head_dim)
    if case.varlen:
        return oracle.prefill_varlen(q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, scale=scale,
                                     causal=case.causal, window=case.window, softcap=case.softcap,
                                     seqs=seqs, rows_per_seq=rows, heads=heads, sink=_f64(sinks))
    return oracle.prefill_dense(q, k, v, scale=scale, causal=case.causal, window=case.window,
                                softcap=case.softcap, q_rows=rows, heads=heads, sink=_f64(sinks))


def _f64(sinks):
    """The sink logits as the kernels receive them (float32), widened."""
    return None if sinks is None else np.asarray(sinks, dtype=np.float32).astype(np.float64)


def check_prefill_full(case, label: str, sinks=None) -> dict:
    """Every output of a small case against the oracle."""
    note(f"[prefill] {label}: B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
         f"Nq={case.seqlen_q} Nk={case.seqlen_k} D={case.head_dim} {case.dtype} causal={case.causal} "
         f"window={case.window} softcap={case.softcap} varlen={case.varlen}")
    o, lse = run_prefill(case, sinks=sinks)
    ro, rl = oracle_prefill(case, sinks=sinks)
    s1 = compare(widen(o, case.dtype), ro, case.dtype, f"{label} O")
    s2 = compare(lse.numpy(), rl, case.dtype, f"{label} LSE", lse=True)
    return {**s1, "lse_max_abs": s2["max_abs"]}


def check_prefill_sampled(case, label: str, *, rows, heads, batches=None) -> dict:
    """Full-size case: the GPU computes everything, the oracle a sample of rows."""
    note(f"[prefill-sampled] {label}")
    o, lse = run_prefill(case)
    rows = np.asarray(rows)
    heads = np.asarray(heads)
    stats = {}
    if case.varlen:
        seqs = list(range(case.batch)) if batches is None else list(batches)
        per = {}
        for b in seqs:
            L = int(case.cu_seqlens_q[b + 1] - case.cu_seqlens_q[b])
            per[b] = np.unique(np.clip(rows, 0, L - 1))
        ro, rl = oracle_prefill(case, rows=per, heads=heads, seqs=seqs)
        for b in seqs:
            tok = case.cu_seqlens_q[b] + per[b]
            g_o = widen(o[tok][:, heads], case.dtype)
            stats[b] = compare(g_o, ro[tok][:, heads], case.dtype, f"{label} seq {b} O")
            compare(lse.numpy()[heads][:, tok], rl[heads][:, tok], case.dtype, f"{label} seq {b} LSE",
                    lse=True)
        return stats
    batches = range(case.batch) if batches is None else batches
    ro, rl = oracle_prefill(case, rows=rows, heads=heads)
    for b in batches:
        g_o = widen(o[b][heads][:, rows], case.dtype)
        stats[b] = compare(g_o, ro[b], case.dtype, f"{label} batch {b} O")
        compare(lse.numpy()[b][heads][:, rows], rl[b], case.dtype, f"{label} batch {b} LSE", lse=True)
    return stats


# ----------------------------------------------------------------------------- decode ----

def decode_tensors(case):
    t = dict(q=case.q.cuda(), k_cache=case.k_cache.cuda(), v_cache=case.v_cache.cuda(),
             block_table=torch.from_numpy(case.block_table).cuda(),
             seq_lens=torch.from_numpy(case.seq_lens).cuda())
    if case.k_scale is not None:
        t["k_scale"] = torch.from_numpy(case.k_scale).cuda()
        t["v_scale"] = torch.from_numpy(case.v_scale).cuda()
    return t


def run_decode(case, tensors=None, *, num_splits=0, sinks=None):
    import attention_forward_03_amd as attn
    t = decode_tensors(case) if tensors is None else tensors
    # O and LSE start as NaN inside NaN guard bands (the caching allocator would otherwise
    # hand a call the previous call's block, and rows a plan left unwritten could pass)
    go = Guarded(t["q"].shape, t["q"].dtype)
    gl = Guarded((t["q"].shape[0], t["q"].shape[1]), torch.float32)
    o, lse = attn.decode_paged(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"],
                               case.max_seq_len, k_scale=t.get("k_scale"), v_scale=t.get("v_scale"),
                               num_splits=num_splits, return_lse=True, sinks=_dev_sinks(sinks),
                               out=go.t, lse_out=gl.t)
    torch.cuda.synchronize()
    assert o.data_ptr() == go.t.data_ptr() and lse.data_ptr() == gl.t.data_ptr()
    go.check_guards("decode O")
    gl.check_guards("decode LSE")
    return o.cpu(), lse.cpu()


def oracle_decode(case, seqs=None, sinks=None):
    q = oracle.tensor_to_f64(case.q, case.q_dtype)
    seqs = np.arange(case.num_seqs) if seqs is None else np.asarray(seqs)
    # widen only the pages the sampled sequences use
    pages = np.unique(np.concatenate([case.block_table[s, :(int(case.seq_lens[s]) + 15) // 16]
                                      for s in seqs]))
    remap = np.full(case.k_cache.shape[0], -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    idx = torch.from_numpy(pages).long()
    kc = oracle.tensor_to_f64(case.k_cache[idx], case.kv_dtype)
    vc = oracle.tensor_to_f64(case.v_cache[idx], case.kv_dtype)
    bt = case.block_table.astype(np.int64).copy()
    sub_bt = np.where(bt >= 0, remap[bt], -1)
    return oracle.decode_paged(q, kc, vc, sub_bt, case.seq_lens, scale=oracle.default_scale(case.head_dim),
                               k_scale=case.k_scale, v_scale=case.v_scale, seqs=seqs, sink=_f64(sinks))


def decode_kind(case) -> str:
    return "fp8_e4m3" if case.kv_dtype == "fp8_e4m3" else case.q_dtype


# -------------------------------------------------------------- chunked prefill (paged) ----

def paged_prefill_tensors(case):
    c = case.cache
    return dict(q=case.q.cuda(), k_cache=c.k_cache.cuda(), v_cache=c.v_cache.cuda(),
                block_table=torch.from_numpy(c.block_table).cuda(),
                cu_seqlens_q=torch.from_numpy(case.cu_seqlens_q).cuda(),
                seq_lens_k=torch.from_numpy(c.seq_lens).cuda())


def run_paged_prefill(case, tensors=None, *, gather=True, sinks=None):
    """gather=True: the gathered-key route where the library has one (head_dim 128);
    gather=False: the kernel that reads the pages in place."""
    import attention_forward_03_amd as attn
    t = paged_prefill_tensors(case) if tensors is None else tensors
    o, lse = attn.fwd_paged(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["cu_seqlens_q"],
                            t["seq_lens_k"], case.max_seqlen_q, causal=case.causal, window=case.window,
                            softcap=case.softcap, return_lse=True, gather=gather, sinks=_dev_sinks(sinks),
                            out=torch.full(t["q"].shape, float("nan"), dtype=t["q"].dtype, device=t["q"].device))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_paged_prefill(case, *, seqs=None, rows_per_seq=None, heads=None, sinks=None):
    """Oracle O [T, Hq, D] / LSE [Hq, T] (float64) of a chunked-prefill case; only the pages
    of the sampled sequences are widened."""
    c = case.cache
    nseq = len(case.cu_seqlens_q) - 1
    sel = np.arange(nseq) if seqs is None else np.asarray(seqs)
    used = [c.block_table[s, :(int(c.seq_lens[s]) + 15) // 16] for s in sel]
    pages = np.unique(np.concatenate(used)) if used else np.zeros(0, dtype=np.int64)
    remap = np.zeros(c.k_cache.shape[0], dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    idx = torch.from_numpy(pages.astype(np.int64))
    kc = oracle.tensor_to_f64(c.k_cache[idx], c.kv_dtype)
    vc = oracle.tensor_to_f64(c.v_cache[idx], c.kv_dtype)
    bt = remap[c.block_table.astype(np.int64)]
    q = oracle.tensor_to_f64(case.q, c.q_dtype)
    return oracle.prefill_paged(q, kc, vc, bt, case.cu_seqlens_q, c.seq_lens,
                                scale=oracle.default_scale(c.head_dim), causal=case.causal,
                                window=case.window, softcap=case.softcap,
                                seqs=None if seqs is None else list(sel), rows_per_seq=rows_per_seq,
                                heads=heads, sink=_f64(sinks))
