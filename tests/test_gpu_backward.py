"""GPU parity of the attention backward (dQ, dK, dV) through the C ABI, against the oracle's
derivatives of the definition, on the forward's own O and LSE."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import Guarded, compare, note, widen

pytestmark = pytest.mark.gpu


def _run(case, dout, sinks=None):
    import attention_forward_03_amd as attn
    q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
    kw = dict(causal=case.causal, window=case.window, softcap=case.softcap)
    o, lse = attn.fwd(q, k, v, return_lse=True, sinks=None if sinks is None else torch.as_tensor(sinks).cuda(), **kw)
    # gradients start as NaN inside NaN guard bands: an entry left unwritten fails the
    # comparison, a write past either end changes a guard
    g = [Guarded(x.shape, x.dtype) for x in (q, k, v)]
    dq, dk, dv = attn.bwd(q, k, v, o, dout.cuda(), lse, dq_out=g[0].t, dk_out=g[1].t, dv_out=g[2].t, **kw)
    torch.cuda.synchronize()
    for name, gg in zip(("dQ", "dK", "dV"), g):
        gg.check_guards(name)
    return dq.cpu(), dk.cpu(), dv.cpu()


def _oracle(case, dout, sinks=None):
    q, k, v = (oracle.tensor_to_f64(t, case.dtype) for t in (case.q, case.k, case.v))
    do = oracle.tensor_to_f64(dout, case.dtype)
    return oracle.prefill_backward_dense(q, k, v, do, scale=oracle.default_scale(case.head_dim), causal=case.causal,
                                         window=case.window, softcap=case.softcap,
                                         sink=None if sinks is None else np.asarray(sinks, np.float64))


# Each gradient entry is a sum of products (dV_jd = sum_i P_ij dO_id, dQ_id = sum_j dS_ij K_jd,
# dK_jd = sum_i dS_ij Q_id) whose terms carry the 16-bit rounding of P and dS (2^-9 each),
# and dS also the error of Delta = rowsum(dO O) taken from the forward's 16-bit O (counted
# as P sum_d |dO| |O| per term); the terms can cancel, so the error scales with the sum of
# their magnitudes M, not with the result: |err| <= 2^-7 M + 2^-8 |ref| + 1e-3 per entry.
def _term_magnitudes(case, dout, sinks=None):
    q, k, v = (oracle.tensor_to_f64(t, case.dtype) for t in (case.q, case.k, case.v))
    do = oracle.tensor_to_f64(dout, case.dtype)
    scale = oracle.default_scale(case.head_dim)
    g = case.num_q_heads // case.num_kv_heads
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    nq, nk = case.seqlen_q, case.seqlen_k
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    allowed = np.ones((nq, nk), dtype=bool)
    if case.causal:
        allowed &= j <= i + (nk - nq)
    if case.window > 0:
        allowed &= j > i + (nk - nq) - case.window
    for b in range(case.batch):
        o, lse = oracle.sdpa_fp64(q[b], k[b], v[b], scale=scale, causal=case.causal, window=case.window,
                                  softcap=case.softcap, sink=None if sinks is None else np.asarray(sinks, np.float64))
        for h in range(case.num_q_heads):
            kv = h // g
            s_raw = q[b, h] @ k[b, kv].T
            t = np.tanh(s_raw * scale / case.softcap) if case.softcap > 0 else None
            s = case.softcap * t if t is not None else s_raw * scale
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.where(allowed & np.isfinite(lse[h])[:, None], np.exp(s - lse[h][:, None]), 0.0)
            dp = do[b, h] @ v[b, kv].T
            delta = (do[b, h] * o[h]).sum(axis=1)
            chain = scale * ((1 - t * t) if t is not None else 1.0)
            # Delta is taken from the forward's 16-bit O (its rounding and the forward's own
            # error), which moves dS by P |dO| |O|-sized amounts even where dP - Delta cancels
            e_delta = (np.abs(do[b, h]) * np.abs(o[h])).sum(axis=1)
            ds = (np.abs(p * (dp - delta[:, None])) + p * e_delta[:, None]) * chain
            mv[b, kv] += p.T @ np.abs(do[b, h])
            mq[b, h] = ds @ np.abs(k[b, kv])
            mk[b, kv] += ds.T @ np.abs(q[b, h])
    return mq, mk, mv


def _check(case, label, sinks=None, seed=0):
    note(f"[bwd] {label}")
    dout = workloads.make_grad_out(case.q.shape, dtype=case.dtype, seed=seed + 1)
    got = _run(case, dout, sinks)
    ref = _oracle(case, dout, sinks)
    mags = _term_magnitudes(case, dout, sinks)
    for name, g, r, m in zip(("dQ", "dK", "dV"), got, ref, mags):
        gw = widen(g, case.dtype)
        s = compare(gw, r, "grad", f"{label} {name}")
        err = np.abs(gw - r)
        bound = 2.0 ** -7 * m + 2.0 ** -8 * np.abs(r) + 1e-3
        worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        assert (err <= bound).all(), f"{label} {name}: error {err[worst]:.3e} over {bound[worst]:.3e} at {worst}"
        s["bound_use"] = float((err / bound).max())
        note(f"  {name} {s}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(causal=True, window=50), dict(softcap=20.0)],
                         ids=["full", "causal", "window", "softcap"])
def test_small_bf16(d, mask):
    case = workloads.make_prefill(batch=2, num_q_heads=4, num_kv_heads=2, seqlen_q=200, head_dim=d, dtype="bf16",
                                  seed=d + 60, **mask)
    _check(case, f"D={d} {mask}", seed=d)


def test_f16_and_unequal_lengths():
    case = workloads.make_prefill(batch=1, num_q_heads=4, num_kv_heads=4, seqlen_q=100, seqlen_k=300, head_dim=128,
                                  dtype="f16", seed=61, causal=True)
    _check(case, "f16 Nq < Nk", seed=3)
    # Nq > Nk: the first rows see no key (O = 0, LSE = -inf, no gradient)
    case = workloads.make_prefill(batch=1, num_q_heads=2, num_kv_heads=1, seqlen_q=300, seqlen_k=100, head_dim=128,
                                  dtype="bf16", seed=62, causal=True)
    _check(case, "Nq > Nk", seed=4)


def test_gqa_group_of_eight_and_sink():
    case = workloads.make_prefill(batch=1, num_q_heads=8, num_kv_heads=1, seqlen_q=257, head_dim=128, dtype="bf16",
                                  seed=63, causal=True)
    _check(case, "Hq=8 Hkv=1", seed=5)
    _check(case, "Hq=8 Hkv=1 sink", sinks=np.linspace(-1.0, 4.0, 8).astype(np.float32), seed=6)


@pytest.mark.parametrize("batch,heads,seqlen,chunks", [(4, 16, 512, 1), (2, 16, 384, 3)], ids=["one_chunk", "three_chunks"])
def test_split_of_the_key_blocks(batch, heads, seqlen, chunks):
    """The dK / dV work of a key block runs as one to four chunks, chosen so that a chunk is
    no longer than one CU's share of all the steps (256 CUs): with units x key blocks = 256
    (full mask) the split is 1 chunk, with 96 it is 3 (4 and 2 are covered by the other
    cases: the small shapes and the benchmark's shape)."""
    units, kblocks = batch * heads, (seqlen + 127) // 128
    assert -(-256 // (units * kblocks)) == chunks
    case = workloads.make_prefill(batch=batch, num_q_heads=2 * heads, num_kv_heads=heads, seqlen_q=seqlen,
                                  head_dim=64, dtype="bf16", seed=65 + chunks)
    _check(case, f"{chunks} chunk(s)", seed=8 + chunks)


def test_deterministic():
    """dQ, dK and dV are repeatable bit for bit (the chunked dK / dV partials are summed in a
    fixed order); the query length gives several chunks per key block."""
    case = workloads.make_prefill(batch=1, num_q_heads=4, num_kv_heads=2, seqlen_q=1333, head_dim=128,
                                  dtype="bf16", seed=64, causal=True)
    dout = workloads.make_grad_out(case.q.shape, seed=7)
    a = _run(case, dout)
    b = _run(case, dout)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bench_shape_sampled():
    """The shape the benchmark times (causal GQA B=1 Hq=32 Hkv=8 N=4096 D=128 bf16): the
    oracle takes KV head 0 with its four query heads (dK and dV of a KV head need all of
    them) and the check samples rows of dQ and keys of dK, dV."""
    case = workloads.config_backward()
    dout = workloads.make_grad_out(case.q.shape, seed=11)
    dq, dk, dv = _run(case, dout)
    q, k, v = (oracle.tensor_to_f64(t, "bf16") for t in (case.q[:, :4], case.k[:, :1], case.v[:, :1]))
    do = oracle.tensor_to_f64(dout[:, :4], "bf16")
    rq, rk, rv = oracle.prefill_backward_dense(q, k, v, do, scale=oracle.default_scale(128), causal=True)
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    # full-size: the Frobenius bound and the outer element bound of the "grad" tolerance
    compare(widen(dq[:, :4][:, :, rows], "bf16"), rq[:, :, rows], "grad", "bench dQ")
    compare(widen(dk[:, :1][:, :, rows], "bf16"), rk[:, :, rows], "grad", "bench dK")
    compare(widen(dv[:, :1][:, :, rows], "bf16"), rv[:, :, rows], "grad", "bench dV")
    assert all(torch.isfinite(t.float()).all() for t in (dq, dk, dv))
