"""GPU parity of the persistent form of the head_dim-128 prefill: dense batches with more
work items (256-row query tiles x heads x batch) than the GPU has compute units, so one
workgroup per CU runs several items in turn (items change inside one kernel: the next
item's Q and first K/V tiles load while the current one ends)."""
import zlib

import numpy as np
import pytest
import torch

import workloads
from gpu_support import check_prefill_full, note, oracle_prefill, run_prefill, widen

pytestmark = pytest.mark.gpu


def _items(b, hq, nq):
    return b * hq * ((nq + 255) // 256)


CASES = [  # (dtype, batch, Hq, Hkv, Nq, Nk, causal, window, softcap)
    ("bf16", 2, 64, 8, 640, 640, False, 0, 0.0),     # no mask at all
    ("f16", 2, 64, 8, 640, 640, False, 0, 0.0),
    ("bf16", 2, 96, 8, 300, 512, False, 0, 0.0),     # a partial last query tile
    ("f16", 2, 48, 16, 700, 700, True, 0, 0.0),      # causal
    ("bf16", 2, 48, 16, 700, 700, True, 200, 0.0),   # causal + window
    ("bf16", 3, 48, 6, 520, 520, False, 0, 20.0),    # softcap
    ("f16", 2, 48, 12, 600, 600, True, 64, 10.0),    # causal + window + softcap
    ("bf16", 1, 64, 8, 1100, 300, True, 0, 0.0),     # causal, Nq > Nk: items without keys
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-Hq{c[2]}-Nq{c[4]}-Nk{c[5]}-c{int(c[6])}-w{c[7]}-cap{c[8]:g}"
                                             for c in CASES])
def test_persistent_prefill(case):
    dtype, b, hq, hkv, nq, nk, causal, window, cap = case
    assert _items(b, hq, nq) > 256  # more items than the MI355X's 256 CUs
    c = workloads.make_prefill(batch=b, num_q_heads=hq, num_kv_heads=hkv, seqlen_q=nq, seqlen_k=nk, head_dim=128,
                               dtype=dtype, seed=zlib.crc32(repr(case).encode()), causal=causal, window=window,
                               softcap=cap)
    stats = check_prefill_full(c, f"persistent {case}")
    note(f"  stats {stats}")


def test_persistent_sinks_and_keyless_rows():
    """Per-head sinks (LSE of a row without keys is the sink; O stays 0) in the persistent form."""
    c = workloads.make_prefill(batch=1, num_q_heads=64, num_kv_heads=8, seqlen_q=1100, seqlen_k=300, head_dim=128,
                               dtype="bf16", seed=77, causal=True)
    sinks = np.linspace(-3.0, 4.0, 64).astype(np.float32)
    check_prefill_full(c, "persistent sinks", sinks=sinks)
    o, lse = run_prefill(c, sinks=sinks)
    assert (widen(o, "bf16")[:, :, :800] == 0).all()
    # rows 0..767 form whole items without keys (written outside the loop: the sink itself);
    # rows 768..799 sit in an item with keys, whose epilogue forms the LSE in log2 units
    # (the sink times log2 e, rounded, then times ln 2): within a few ulp
    want = np.repeat(sinks[:, None], 800, axis=1)
    np.testing.assert_array_equal(lse.numpy()[0, :, :768], want[:, :768])
    np.testing.assert_allclose(lse.numpy()[0, :, 768:800], want[:, 768:], rtol=1e-6, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_persistent_dominance_redo_bit_exact(dtype):
    """Dominance probe with 320 items (B=2 Hq=32 N=1280, no mask): targets late in a row beat
    the first sub-tile's reference by more than the slack, so items run their pass again
    inside the persistent loop; every output row must be its target's V row bit for bit."""
    n = 1280
    rng = np.random.default_rng(12)
    targets = rng.integers(0, n, size=n)
    targets[::7] = 0  # some rows whose target is in the first sub-tile
    case = workloads.dominance_prefill(batch=2, num_q_heads=32, num_kv_heads=4, seqlen=n, head_dim=128,
                                       dtype=dtype, targets=targets, seed=43)
    assert _items(2, 32, n) > 256
    o, _ = run_prefill(case)
    group = case.num_q_heads // case.num_kv_heads
    idx = torch.from_numpy(targets).long()
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            want = case.v[b, h // group][idx]
            same = o[b, h].view(torch.int16) == want.view(torch.int16)
            assert bool(same.all()), f"b={b} h={h} first bad row {int((~same.all(1)).nonzero()[0])}"


def test_persistent_deterministic():
    c = workloads.make_prefill(batch=2, num_q_heads=64, num_kv_heads=8, seqlen_q=640, head_dim=128, dtype="bf16",
                               seed=5, causal=True)
    o1, l1 = run_prefill(c)
    o2, l2 = run_prefill(c)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
