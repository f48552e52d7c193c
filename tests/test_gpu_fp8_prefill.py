"""GPU parity of the fp8 (e4m3, per-tensor scales) dense prefill on the fp8 matrix cores,
through the C ABI, against the oracle on the decoded codes."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import compare, note, widen

pytestmark = pytest.mark.gpu


def _run(case, sinks=None, out=None):
    import attention_forward_03_amd as attn
    q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
    if out is None:
        out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    o, lse = attn.fwd(q, k, v, causal=case.causal, window=case.window, softcap=case.softcap, return_lse=True,
                      q_scale=case.q_scale, k_scale=case.k_scale, v_scale=case.v_scale, out=out,
                      sinks=None if sinks is None else torch.as_tensor(sinks).cuda())
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _oracle(case, sinks=None, rows=None, heads=None, abs_v=False):
    qc, kc, vc = (oracle.tensor_to_f64(t, "fp8_e4m3") for t in (case.q, case.k, case.v))
    if abs_v:
        vc = np.abs(vc)
    return oracle.prefill_fp8(qc, kc, vc, q_scale=case.q_scale, k_scale=case.k_scale, v_scale=case.v_scale,
                              scale=oracle.default_scale(case.head_dim), causal=case.causal, window=case.window,
                              softcap=case.softcap, q_rows=rows, heads=heads,
                              sink=None if sinks is None else np.asarray(sinks, np.float64))


# P is rounded to e4m3 and normalised by the sum of the rounded values: with
# p_hat_j = p_j (1 + eps_j) the weights become w_j (1 + eps_j) / (1 + eps_bar),
# eps_bar = sum_j w_j eps_j, and
#   O_gpu - O = sum_j w_j eps_j (v_j - O) / (1 + eps_bar)
# (a sink only rescales every w_j). A normal e4m3 number is off by at most 2^-4 of itself;
# the kernel keeps the row's largest P >= 2^6, so a P in the subnormal range (< 2^-6, steps
# of 2^-9) is off by at most 2^-10, i.e. 2^-16 of the row sum. Hence
#   |O_gpu - O| <= (2^-4 sum_j w_j |v_j - O| + 2^-16 sum_j |v_j - O|) / (1 - 2^-4)
# over the allowed keys, plus the bf16 rounding of O (2^-8 |O|) and fp32 accumulation (1e-3).
K_P = 2.0 ** -4 / (1.0 - 2.0 ** -4)
K_SUB = 2.0 ** -16 / (1.0 - 2.0 ** -4)


def _spread(case, ro, sinks=None):
    """K_P sum_j w_ij |v_j - O_i| + K_SUB sum_j |v_j - O_i| (allowed keys) per output, from
    the scores (small cases)."""
    qc, kc, vc = (oracle.tensor_to_f64(t, "fp8_e4m3") for t in (case.q, case.k, case.v))
    q, k, v = qc * case.q_scale, kc * case.k_scale, vc * case.v_scale
    out = np.zeros_like(ro)
    g = case.num_q_heads // case.num_kv_heads
    nq, nk = case.seqlen_q, case.seqlen_k
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    allowed = np.ones((nq, nk), dtype=bool)
    if case.causal:
        allowed &= j <= i + (nk - nq)
    if case.window > 0:
        allowed &= j > i + (nk - nq) - case.window
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            w = oracle.attention_probs(q[b, h][None], k[b, h // g][None], scale=oracle.default_scale(128),
                                       causal=case.causal, window=case.window, softcap=case.softcap)[0]
            if sinks is not None:
                l0 = _lse_nosink(q[b, h], k[b, h // g], case)
                w = w * np.exp(l0 - np.logaddexp(l0, float(sinks[h])))[:, None]
            dev = np.abs(v[b, h // g][None, :, :] - ro[b, h][:, None, :])      # [Nq, Nk, D]
            out[b, h] = K_P * np.einsum("ij,ijd->id", w, dev) + K_SUB * np.einsum("ij,ijd->id", allowed * 1.0, dev)
    return out


def _lse_nosink(q, k, case):
    _, lse = oracle.sdpa_fp64(q[None], k[None], k[None], scale=oracle.default_scale(128), causal=case.causal,
                              window=case.window, softcap=case.softcap)
    return lse[0]


def _element_bound(o_gpu, ro, spread, what):
    fin = np.isfinite(ro)
    err = np.abs(o_gpu - ro)[fin]
    bound = (spread + 2.0 ** -8 * np.abs(ro) + 1e-3)[fin]
    worst = int(np.argmax(err - bound)) if err.size else 0
    assert (err <= bound).all(), f"{what}: error {err[worst]:.3e} over the bound {bound[worst]:.3e}"
    return float((err / bound).max()) if err.size else 0.0


def _check(case, label, sinks=None):
    note(f"[fp8] {label}")
    o, lse = _run(case, sinks)
    ro, rl = _oracle(case, sinks)
    g = widen(o, "bf16")
    s = compare(g, ro, "fp8_prefill", f"{label} O")
    compare(lse.numpy(), rl, "fp8_prefill", f"{label} LSE", lse=True)
    s["bound_use"] = _element_bound(g, ro, _spread(case, ro, sinks), f"{label} O")
    note(f"  stats {s}")
    return s


@pytest.mark.parametrize("mask", [dict(), dict(causal=True), dict(causal=True, window=77), dict(softcap=20.0)],
                         ids=["full", "causal", "window", "softcap"])
def test_small(mask):
    case = workloads.make_prefill_fp8(batch=2, num_q_heads=4, num_kv_heads=2, seqlen_q=333, head_dim=128,
                                      seed=51, **mask)
    _check(case, f"fp8 {mask}")


def test_shorter_queries_and_keyless_rows():
    case = workloads.make_prefill_fp8(batch=1, num_q_heads=2, num_kv_heads=1, seqlen_q=150, seqlen_k=400,
                                      head_dim=128, seed=52, causal=True)
    _check(case, "fp8 Nq < Nk")
    case = workloads.make_prefill_fp8(batch=1, num_q_heads=2, num_kv_heads=1, seqlen_q=330, seqlen_k=40,
                                      head_dim=128, seed=53, causal=True)
    _check(case, "fp8 Nq > Nk")
    o, lse = _run(case)
    assert (widen(o, "bf16")[:, :, :290] == 0).all()


def test_sharp_attention_and_sink():
    # larger inputs give peaked softmax rows (the opposite regime to near-uniform rows)
    case = workloads.make_prefill_fp8(batch=1, num_q_heads=4, num_kv_heads=4, seqlen_q=300, head_dim=128,
                                      seed=54, input_scale=3.0)
    _check(case, "fp8 sharp")
    _check(case, "fp8 sharp + sink", sinks=np.array([0.5, 3.0, -2.0, 8.0], dtype=np.float32))


def test_deterministic():
    case = workloads.make_prefill_fp8(batch=1, num_q_heads=2, num_kv_heads=2, seqlen_q=700, head_dim=128,
                                      seed=55, causal=True)
    o1, _ = _run(case)
    o2, _ = _run(case)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_headline_shape_sampled():
    """The shape the benchmark times (B=1 H=32 N=8192 D=128, fp8 e4m3 Q/K/V); the oracle
    takes sampled rows of three heads."""
    case = workloads.config_fp8_headline()
    o, lse = _run(case)
    rows = np.array([0, 1, 255, 256, 4097, 8191])
    heads = np.array([0, 13, 31])
    ro, rl = _oracle(case, rows=rows, heads=heads)
    g = widen(o[0][heads][:, rows], "bf16")
    compare(g, ro[0], "fp8_prefill", "fp8 headline O")
    # sum_j w_j |v_j - O| <= sum_j w_j |v_j| + |O| (the oracle on |V|); sum_j |v_j - O| <=
    # N (max |v| + |O|)
    oabs, _ = _oracle(case, rows=rows, heads=heads, abs_v=True)
    vmax = float(np.abs(oracle.tensor_to_f64(case.v, "fp8_e4m3")).max()) * case.v_scale
    spread = K_P * (oabs[0] + np.abs(ro[0])) + K_SUB * case.seqlen_k * (vmax + np.abs(ro[0]))
    _element_bound(g, ro[0], spread, "fp8 headline O")
    compare(lse.numpy()[0][heads][:, rows], rl[0], "fp8_prefill", "fp8 headline LSE", lse=True)
    assert torch.isfinite(o.float()).all()
