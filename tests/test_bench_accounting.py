"""CPU checks of the work bench.py divides its timings by: the allowed (query, key) pairs
against the oracle's own mask, the FLOPs of a prefill against a count of the
multiply-adds of the definition, the chunked prefill's FLOPs against the mask of every
chunk, and the decode's algorithmic bytes against a token-by-token count of what a decode
has to read and write. No GPU."""
import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402
from oracle.attention import _allowed  # noqa: E402


def _oracle_pairs(nq, nk, causal, window):
    m = _allowed(nq, nk, causal=causal, window=window, q_pos=np.arange(nq), nq_total=nq)
    return nq * nk if m is None else int(np.count_nonzero(m))


@pytest.mark.parametrize("nq,nk", [(1, 1), (7, 7), (64, 64), (100, 37), (37, 100), (300, 1000), (1000, 300)])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 1), (True, 16), (True, 5000)])
def test_allowed_pairs_match_the_oracle_mask(nq, nk, causal, window):
    assert bench.allowed_pairs(nq, nk, causal, window) == _oracle_pairs(nq, nk, causal, window)


def test_prefill_flops_count_two_products():
    # S = Q K^T and O = P V, each nq * nk * d multiply-adds per (batch, head), 2 FLOPs each
    b, h, nq, nk, d = 2, 3, 5, 7, 4
    mads = 0
    for _ in range(b * h):
        for _i in range(nq):
            for _j in range(nk):
                mads += d  # one score
                mads += d  # its share of the output row
    assert bench.prefill_flops(b, h, nq, nk, d) == 2 * mads


def test_chunked_flops_follow_each_chunks_mask():
    case = workloads.make_paged_prefill(lengths_q=[5, 40, 1], lengths_k=[5, 123, 70], num_q_heads=4, num_kv_heads=2,
                                        head_dim=64, seed=3, causal=True, window=50)
    nq = np.diff(case.cu_seqlens_q)
    pairs = sum(_oracle_pairs(int(a), int(b), True, 50) for a, b in zip(nq, case.seq_lens_k))
    assert bench.chunked_flops(case) == 4.0 * 64 * 4 * pairs


@pytest.mark.parametrize("kv,elt", [("bf16", 2), ("fp8_e4m3", 1)])
def test_decode_bytes_count_every_row_read_once(kv, elt):
    case = workloads.make_decode(lengths=[1, 17, 700], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                 kv_dtype=kv, seed=1)
    total = 0
    for length in case.seq_lens:
        for _t in range(int(length)):
            for _g in range(case.num_kv_heads):
                total += 2 * case.head_dim * elt                      # its K row and its V row
        total += 4 * math.ceil(int(length) / 16) + 4                  # block-table entries, length
    total += 2 * len(case.seq_lens) * case.num_q_heads * case.head_dim * 2   # Q read, O written
    if kv == "fp8_e4m3":
        total += 2 * case.num_kv_heads * 4                            # k_scale, v_scale
    assert bench.decode_bytes(case, kv_elt=elt) == total
