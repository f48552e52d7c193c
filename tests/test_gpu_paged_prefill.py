"""GPU parity of attn_fwd_paged (chunked prefill over the paged KV cache, through the C ABI).

Unused block-table entries and the slots past each sequence's last key hold NaN pages
(the generator's poison), so a kernel that reads outside a sequence's keys fails the
finiteness check of every comparison.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_support import (compare, note, oracle_paged_prefill, paged_prefill_tensors, run_paged_prefill,
                         run_prefill, widen)

pytestmark = pytest.mark.gpu

# chunk lengths / key lengths: page tails, a chunk equal to its keys, a one-token chunk, and
# chunks shorter than one 256-row block and longer
LENS_Q = [1, 17, 300, 64, 5, 129]
LENS_K = [1, 40, 700, 64, 261, 1029]
MASKS = [dict(causal=True), dict(causal=False), dict(causal=True, window=37), dict(causal=True, softcap=5.0)]


def _case(dtype, d, hq, hkv, mask, seed, lens_q=LENS_Q, lens_k=LENS_K):
    return workloads.make_paged_prefill(lengths_q=lens_q, lengths_k=lens_k, num_q_heads=hq, num_kv_heads=hkv,
                                        head_dim=d, dtype=dtype, seed=seed, **mask)


def _check(case, label, gather=True):
    note(f"[paged-prefill] {label} gather={gather}")
    o, lse = run_paged_prefill(case, gather=gather)
    ro, rl = oracle_paged_prefill(case)
    s = compare(widen(o, case.cache.q_dtype), ro, case.cache.q_dtype, f"{label} O")
    compare(lse.numpy(), rl, case.cache.q_dtype, f"{label} LSE", lse=True)
    note(f"  stats {s}")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=["causal", "full", "window", "softcap"])
def test_small_bf16(d, mask):
    _check(_case("bf16", d, 8, 2, mask, seed=d), f"bf16 D={d} {mask}")


@pytest.mark.parametrize("mask", MASKS, ids=["causal", "full", "window", "softcap"])
def test_small_bf16_d128_pages_in_place(mask):
    """head_dim 128 without a workspace: the kernel that reads the pages in place."""
    _check(_case("bf16", 128, 8, 2, mask, seed=128), f"bf16 D=128 {mask}", gather=False)


def test_routes_agree_and_gather_is_repeatable():
    case = _case("bf16", 128, 8, 2, dict(causal=True, window=300), seed=129)
    t = paged_prefill_tensors(case)
    o_g, l_g = run_paged_prefill(case, t, gather=True)
    o_d, l_d = run_paged_prefill(case, t, gather=False)
    compare(widen(o_g, "bf16"), widen(o_d, "bf16"), "bf16", "gathered vs in-place O")
    compare(l_g.numpy(), l_d.numpy(), "bf16", "gathered vs in-place LSE", lse=True)
    o_g2, _ = run_paged_prefill(case, t, gather=True)
    assert torch.equal(o_g.view(torch.int16), o_g2.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_small_f16(d):
    _check(_case("f16", d, 4, 4, dict(causal=True), seed=100 + d), f"f16 D={d}")


@pytest.mark.parametrize("heads", [(32, 8), (16, 1), (2, 2)])
def test_gqa_and_mqa(heads):
    hq, hkv = heads
    _check(_case("bf16", 128, hq, hkv, dict(causal=True), seed=200 + hq), f"heads {heads}")


def test_more_queries_than_keys_and_empty_sequences():
    # causal with Nq > Nk: the first Nq - Nk rows see no key (O = 0, LSE = -inf); a sequence
    # with no keys at all; an empty chunk
    case = _case("bf16", 128, 4, 2, dict(causal=True), seed=300, lens_q=[10, 3, 0, 7], lens_k=[4, 0, 5, 7])
    _check(case, "Nq > Nk, Nk = 0, Nq = 0")
    case = _case("bf16", 64, 4, 2, dict(causal=False), seed=301, lens_q=[3, 6], lens_k=[0, 20])
    _check(case, "non-causal, Nk = 0")


def test_equals_ragged_prefill_bitwise():
    """With each chunk equal to its whole sequence the paged form computes the same
    products in the same order as the ragged attn_fwd of the same kernel family (D = 64):
    the results agree bit for bit."""
    lens = [300, 17, 1029, 64]
    case = workloads.make_paged_prefill(lengths_q=lens, lengths_k=lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                                        dtype="bf16", seed=400, causal=True, window=100, keep_logical=True)
    o_p, l_p = run_paged_prefill(case)
    # the same keys as packed [T, Hkv, D] tensors
    kv = [torch.cat(x) for x in (case.cache.k_logical, case.cache.v_logical)]
    cu = case.cu_seqlens_q
    rag = workloads.PrefillCase(q=case.q, k=kv[0], v=kv[1], batch=len(lens), num_q_heads=8, num_kv_heads=2,
                                seqlen_q=max(lens), seqlen_k=max(lens), head_dim=64, dtype="bf16", causal=True,
                                window=100, cu_seqlens_q=cu, cu_seqlens_k=cu)
    o_r, l_r = run_prefill(rag)
    assert torch.equal(o_p.view(torch.int16), o_r.view(torch.int16))
    assert torch.equal(l_p, l_r)


@pytest.mark.parametrize("gather", [True, False], ids=["gathered", "in-place"])
def test_chunked_prefill_workload_sampled(gather):
    """The workload the benchmark times (8 chunks of 2048 queries over contexts up to 14336
    keys, Hq=32, Hkv=8, D=128, bf16), in the same launches; the oracle takes sampled rows of
    three sequences, among them the first and last rows of each chunk."""
    case = workloads.config_chunked_prefill()
    note(f"[paged-prefill] workload: keys {case.seq_lens_k.tolist()} gather={gather}")
    t = paged_prefill_tensors(case)
    o, lse = run_paged_prefill(case, t, gather=gather)
    seqs = [0, 3, 7]
    rows = {s: np.unique(np.r_[0, 1, 255, 256, 1000, 2046, 2047]) for s in seqs}
    heads = np.array([0, 5, 31])
    ro, rl = oracle_paged_prefill(case, seqs=seqs, rows_per_seq=rows, heads=heads)
    for s in seqs:
        tok = case.cu_seqlens_q[s] + rows[s]
        compare(widen(o[tok][:, heads], "bf16"), ro[tok][:, heads], "bf16", f"workload seq {s} O")
        compare(lse.numpy()[heads][:, tok], rl[heads][:, tok], "bf16", f"workload seq {s} LSE", lse=True)
    # and every output is finite
    assert torch.isfinite(o.float()).all()
