"""GPU parity of the 16-bit prefill at head dims 96, 192 and 256 (padded LDS rows for 96
and 192; 4-wave workgroups for 192 and 256), dense, masked, ragged, with a sink, and as
chunked prefill over the paged cache, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads
from gpu_support import (check_prefill_full, check_prefill_sampled, compare, note, oracle_paged_prefill,
                         run_paged_prefill, run_prefill, widen)

pytestmark = pytest.mark.gpu

DIMS = [96, 192, 256]
MASKS = [dict(), dict(causal=True), dict(causal=True, window=77), dict(softcap=15.0)]
MASK_IDS = ["full", "causal", "window", "softcap"]


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("mask", MASKS, ids=MASK_IDS)
def test_dense_bf16(d, mask):
    # lengths with tails in every tile size (64 and 32 keys, 128 and 256 rows)
    case = workloads.make_prefill(batch=2, num_q_heads=4, num_kv_heads=2, seqlen_q=333, seqlen_k=333,
                                  head_dim=d, dtype="bf16", seed=d, **mask)
    check_prefill_full(case, f"D={d} {mask}")


@pytest.mark.parametrize("d", DIMS)
def test_f16_and_shorter_queries(d):
    case = workloads.make_prefill(batch=1, num_q_heads=4, num_kv_heads=1, seqlen_q=150, seqlen_k=400,
                                  head_dim=d, dtype="f16", seed=d + 1, causal=True)
    check_prefill_full(case, f"f16 D={d} Nq<Nk")


@pytest.mark.parametrize("d", DIMS)
def test_ragged_and_sink(d):
    case = workloads.make_prefill_varlen(lengths_q=[300, 1, 77, 520], num_q_heads=4, num_kv_heads=2, head_dim=d,
                                         dtype="bf16", seed=d + 2, causal=True)
    sinks = np.random.default_rng(d).uniform(-2, 6, size=4).astype(np.float32)
    check_prefill_full(case, f"ragged D={d}")
    check_prefill_full(case, f"ragged sink D={d}", sinks=sinks)


@pytest.mark.parametrize("d", DIMS)
def test_dominance_probe_bit_exact(d):
    n = 300
    targets = np.random.default_rng(d).integers(0, n, size=n)
    for kw in (dict(), dict(causal=True)):
        t = np.minimum(targets, np.arange(n)) if kw else targets
        case = workloads.dominance_prefill(batch=1, num_q_heads=2, num_kv_heads=1, seqlen=n, head_dim=d,
                                           dtype="bf16", targets=t, seed=43, **kw)
        o, _ = run_prefill(case)
        want = case.v[0, 0][torch.from_numpy(t).long()]
        for h in range(2):
            assert torch.equal(o[0, h].view(torch.int16), want.view(torch.int16)), (d, kw, h)


@pytest.mark.parametrize("d", DIMS)
def test_chunked_prefill_in_place(d):
    case = workloads.make_paged_prefill(lengths_q=[17, 300, 1, 64], lengths_k=[40, 700, 1, 64], num_q_heads=8,
                                        num_kv_heads=2, head_dim=d, dtype="bf16", seed=d + 3, window=100)
    o, lse = run_paged_prefill(case)
    ro, rl = oracle_paged_prefill(case)
    compare(widen(o, "bf16"), ro, "bf16", f"chunked D={d} O")
    compare(lse.numpy(), rl, "bf16", f"chunked D={d} LSE", lse=True)


@pytest.mark.parametrize("d", DIMS)
def test_bench_shape_sampled(d):
    """The shape the benchmark times for these head dims: B=2 H=16 N=4096, bf16, causal."""
    case = workloads.config_headdim(d)
    note(f"[headdim] D={d} sampled")
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    check_prefill_sampled(case, f"D={d} N=4096", rows=rows, heads=np.array([0, 9, 15]), batches=[1])
