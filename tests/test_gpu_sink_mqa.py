"""GPU parity of the attention sink (every prefill kernel, the chunked prefill and the
decode combine) and of decode with more than 16 query heads per KV head (MQA-like
groups), through the C ABI."""
import numpy as np
import pytest
import torch

import workloads
from gpu_support import (check_prefill_full, compare, decode_kind, note, oracle_decode, oracle_paged_prefill,
                         run_decode, run_paged_prefill, run_prefill, widen)

pytestmark = pytest.mark.gpu


def _sinks(hq, seed, spread=3.0):
    # logits around the size of typical row LSEs, so the sink takes a visible share
    return np.random.default_rng(seed).uniform(-spread, spread + 4.0, size=hq).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_prefill_sink_dense(dtype, d):
    case = workloads.make_prefill(batch=2, num_q_heads=4, num_kv_heads=2, seqlen_q=300, seqlen_k=300,
                                  head_dim=d, dtype=dtype, seed=d + 7)
    check_prefill_full(case, f"sink dense {dtype} D={d}", sinks=_sinks(4, d))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mask", [dict(causal=True), dict(causal=True, window=50), dict(causal=True, softcap=20.0)],
                         ids=["causal", "window", "softcap"])
def test_prefill_sink_masked_with_keyless_rows(dtype, mask):
    # Nq - Nk = 330 > 256: rows without keys (a whole 256-row block at D = 128) get O = 0, LSE = sink
    case = workloads.make_prefill(batch=1, num_q_heads=4, num_kv_heads=1, seqlen_q=400, seqlen_k=70,
                                  head_dim=128, dtype=dtype, seed=11, **mask)
    sinks = _sinks(4, 12)
    check_prefill_full(case, f"sink {dtype} {mask}", sinks=sinks)
    o, lse = run_prefill(case, sinks=sinks)
    assert (widen(o, dtype)[:, :, :330] == 0).all()
    np.testing.assert_allclose(lse.numpy()[0, :, :330], np.repeat(sinks[:, None], 330, axis=1), rtol=1e-6)


def test_prefill_sink_ragged():
    case = workloads.make_prefill_varlen(lengths_q=[300, 7, 520], lengths_k=[300, 0, 900], num_q_heads=8,
                                         num_kv_heads=2, head_dim=128, dtype="bf16", seed=13, causal=True)
    check_prefill_full(case, "sink ragged", sinks=_sinks(8, 14))


def test_prefill_negligible_sink_is_no_sink():
    case = workloads.make_prefill(batch=1, num_q_heads=4, num_kv_heads=4, seqlen_q=513, seqlen_k=513,
                                  head_dim=128, dtype="bf16", seed=15, causal=True)
    o0, l0 = run_prefill(case)
    o1, l1 = run_prefill(case, sinks=np.full(4, -1e30, dtype=np.float32))
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)


@pytest.mark.parametrize("gather", [True, False], ids=["gathered", "in-place"])
def test_chunked_prefill_sink(gather):
    case = workloads.make_paged_prefill(lengths_q=[17, 300, 1], lengths_k=[40, 700, 1], num_q_heads=8,
                                        num_kv_heads=2, head_dim=128, dtype="bf16", seed=16)
    sinks = _sinks(8, 17)
    o, lse = run_paged_prefill(case, gather=gather, sinks=sinks)
    ro, rl = oracle_paged_prefill(case, sinks=sinks)
    compare(widen(o, "bf16"), ro, "bf16", "chunked sink O")
    compare(lse.numpy(), rl, "bf16", "chunked sink LSE", lse=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
# (32, 1): one wave takes both 16-head tiles; (20, 1): its second tile holds 4 heads;
# (48, 1): three tiles, so the second wave's second tile is empty; (64, 4): 16 heads, one tile
@pytest.mark.parametrize("heads", [(32, 1), (20, 1), (48, 1), (48, 2), (64, 4)])
def test_decode_many_heads_per_kv_head(kv, heads):
    hq, hkv = heads
    case = workloads.make_decode(lengths=[1, 17, 1000, 4099], num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                 kv_dtype=kv, seed=hq + hkv)
    note(f"[decode] Hq={hq} Hkv={hkv} {kv}")
    for ns in (0, 3):
        o, lse = run_decode(case, num_splits=ns)
        ro, rl = oracle_decode(case)
        compare(widen(o, case.q_dtype), ro, decode_kind(case), f"decode {heads} splits={ns} O")
        compare(lse.numpy(), rl, decode_kind(case), f"decode {heads} splits={ns} LSE", lse=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("hkv", [8, 1], ids=["gqa", "mqa"])
def test_decode_sink(kv, hkv):
    case = workloads.make_decode(lengths=[1, 33, 2000, 5000], num_q_heads=32, num_kv_heads=hkv, head_dim=128,
                                 kv_dtype=kv, seed=21)
    sinks = _sinks(32, 22)
    for ns in (0, 1, 4):
        o, lse = run_decode(case, num_splits=ns, sinks=sinks)
        ro, rl = oracle_decode(case, sinks=sinks)
        compare(widen(o, case.q_dtype), ro, decode_kind(case), f"decode sink splits={ns} O")
        compare(lse.numpy(), rl, decode_kind(case), f"decode sink splits={ns} LSE", lse=True)
