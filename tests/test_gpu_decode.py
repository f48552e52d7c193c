"""GPU parity of attn_decode_paged (split kernel + LSE combine, through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import compare, decode_kind, decode_tensors, note, oracle_decode, run_decode, widen

pytestmark = pytest.mark.gpu

SMALL_LENGTHS = [1, 15, 16, 17, 100, 1000, 4099, 257]


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
# (16, 16), (12, 12), (16, 4), (24, 6): fp8 workgroups of 8, 4, 4 and 2 KV-head waves that
# cover part of the KV heads each (2, 3, 1 and 3 groups per split)
@pytest.mark.parametrize("heads", [(32, 8), (8, 8), (16, 1), (4, 2), (16, 16), (12, 12), (16, 4), (24, 6)])
def test_small_decode(kv, heads):
    hq, hkv = heads
    case = workloads.make_decode(lengths=SMALL_LENGTHS, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                 kv_dtype=kv, seed=hq * 100 + hkv)
    note(f"[decode] small {kv} Hq={hq} Hkv={hkv}")
    o, lse = run_decode(case)
    ro, rl = oracle_decode(case)
    kind = decode_kind(case)
    s = compare(widen(o, case.q_dtype), ro, kind, f"decode {kv} {heads} O")
    compare(lse.numpy(), rl, kind, f"decode {kv} {heads} LSE", lse=True)
    note(f"  stats {s}")


@pytest.mark.parametrize("kv,heads", [("f16", (8, 2)), ("fp8_e4m3", (8, 2)), ("fp8_e4m3", (32, 1)), ("f16", (32, 1))],
                         ids=["f16", "fp8_kv", "fp8_kv_two_tiles", "f16_two_tiles"])
def test_f16_decode(kv, heads):
    """f16 queries, over f16 KV or over fp8 KV (codes widened to f16), with one head tile per
    wave or two."""
    case = workloads.make_decode(lengths=[3, 700, 33], num_q_heads=heads[0], num_kv_heads=heads[1], head_dim=128,
                                 q_dtype="f16", kv_dtype=kv, seed=7)
    o, lse = run_decode(case)
    ro, rl = oracle_decode(case)
    compare(widen(o, "f16"), ro, decode_kind(case), f"decode f16 {kv} O")
    compare(lse.numpy(), rl, decode_kind(case), f"decode f16 {kv} LSE", lse=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_split_invariance(kv):
    case = workloads.make_decode(lengths=[5000, 1, 2048, 3001], num_q_heads=8, num_kv_heads=2,
                                 head_dim=128, kv_dtype=kv, seed=11)
    t = decode_tensors(case)
    ro, rl = oracle_decode(case)
    outs = []
    for ns in (1, 2, 7, 313, 0):
        o, lse = run_decode(case, t, num_splits=ns)
        compare(widen(o, "bf16"), ro, decode_kind(case), f"splits={ns} O")
        compare(lse.numpy(), rl, decode_kind(case), f"splits={ns} LSE", lse=True)
        outs.append(o)
    # repeated calls with the same plan are bitwise identical
    o2, _ = run_decode(case, t, num_splits=7)
    assert torch.equal(outs[2].view(torch.int16), o2.view(torch.int16))


def _probe_case(kv, lengths, targets_fn, hq=8, hkv=2, seed=3):
    case = workloads.make_decode(lengths=lengths, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                 kv_dtype=kv, seed=seed, pow2_scales=True)
    targets = np.stack([targets_fn(int(L), hq) for L in case.seq_lens])
    return workloads.dominance_decode(case, targets), targets


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_dominance_probe_bit_exact(kv, splits):
    """Query (s, h) targets a chosen token; O must equal that V row bit-exactly. Targets sit
    on page and split boundaries, at the first and the last token."""
    lengths = [1, 16, 17, 1000, 4099, 2048, 33]

    def targets(L, hq):
        cand = np.array([0, L - 1, 15, 16, 255, 256, 1023, 1024, L // 2, L - 17])
        return np.clip(cand[np.arange(hq) % len(cand)], 0, L - 1)

    case, tg = _probe_case(kv, lengths, targets)
    o, _ = run_decode(case, num_splits=splits)
    group = case.num_q_heads // case.num_kv_heads
    for s in range(case.num_seqs):
        for h in range(case.num_q_heads):
            t = int(tg[s, h])
            page = int(case.block_table[s, t // 16])
            row = case.v_cache[page, t % 16, h // group].float()
            if case.v_scale is not None:
                row = row * float(case.v_scale[h // group])
            want = row.to(torch.bfloat16)
            got = o[s, h]
            # An exactly-zero target entry (an fp8 code 0) stays a tiny nonzero: the other keys'
            # weights are below e^-45 each, so their sum survives there (correctly) as a value
            # below 1e-30. Every other entry must equal the target row bit for bit.
            nz = want != 0
            assert torch.equal(got.view(torch.int16)[nz], want.view(torch.int16)[nz]), (s, h, t)
            assert bool((got[~nz].float().abs() < 1e-30).all()), (s, h, t)


def test_fp8_all_codes_decode_exactly():
    """Every finite e4m3 code, placed in the V rows a probe selects, comes out as the oracle's
    own table value times the (power-of-two) scale, bit-exactly in bf16."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)  # 254 codes
    case, tg = _probe_case("fp8_e4m3", [40], lambda L, hq: np.array([3, 7] * (hq // 2)), hq=2, hkv=1)
    vc = case.v_cache.view(torch.uint8).clone()
    for t, chunk in ((3, codes[:128]), (7, codes[128:])):
        page = int(case.block_table[0, t // 16])
        row = np.zeros(128, dtype=np.uint8)
        row[:len(chunk)] = chunk
        vc[page, t % 16, 0] = torch.from_numpy(row)
    case.v_cache = vc.view(torch.float8_e4m3fn)
    o, _ = run_decode(case)
    table = oracle.e4m3_code_table() * float(case.v_scale[0])
    for h, (t, chunk) in enumerate(((3, codes[:128]), (7, codes[128:]))):
        got = widen(o[0, h], "bf16")[:len(chunk)]
        want = table[chunk]
        nz = want != 0  # codes 0x00 / 0x80: see the note in test_dominance_probe_bit_exact
        assert np.array_equal(got[nz], want[nz]), (h, got[:8], want[:8])
        assert (np.abs(got[~nz]) < 1e-30).all()


@pytest.mark.parametrize("kv,hkv", [("bf16", 8), ("fp8_e4m3", 8), ("bf16", 1)], ids=["bf16", "fp8_e4m3", "mqa_bf16"])
def test_full_decode_config_sampled(kv, hkv):
    """64 sequences, L ~ U[512, 32768], Hq=32 Hkv=8 D=128 (and the MQA form, Hkv=1, as the
    bench times it): the GPU computes all, the oracle checks the shortest, the longest and a
    few more sequences."""
    case = workloads.config_decode(kv, num_kv_heads=hkv)
    note(f"[decode] full {kv} Hkv={hkv}: total tokens {int(case.seq_lens.sum())}")
    o, lse = run_decode(case)
    order = np.argsort(case.seq_lens)
    seqs = np.unique(np.concatenate([order[:2], order[-2:], [7, 33]]))
    ro, rl = oracle_decode(case, seqs)
    s = compare(widen(o[torch.from_numpy(seqs).long()], "bf16"), ro, decode_kind(case), f"full {kv} O")
    compare(lse.numpy()[seqs], rl, decode_kind(case), f"full {kv} LSE", lse=True)
    note(f"  stats {s}")
