"""LDS bank model of the fp8 prefill tile layout (host only).

The model: 64 banks of 4 bytes; 16-byte reads serve 16 lanes per cycle, 8-byte
transposing reads 32 lanes per cycle; a cycle takes as long as its most-used bank. It
reproduces the bank-conflict counts measured with SQ_LDS_BANK_CONFLICT on MI355X (two
extra cycles per 8-bit transposing read with the row term (k >> 1) & 7; none with the
term whose two low bits are swapped), and it checks that the layout the fp8 kernel uses
(csrc/prefill_fp8.hip: sw8, the K and V^T read addresses) is conflict-free for every
read the kernel issues.
"""
import itertools

import pytest

D = 128  # bytes per LDS row (head_dim 128, one byte per e4m3 code)


def g_old(k):
    return (k >> 1) & 7


def g_new(k):
    x = (k >> 1) & 7
    return (x & 4) | ((x & 1) << 1) | ((x >> 1) & 1)


def extra_cycles(addrs, lanes_per_cycle, nbytes):
    """Cycles beyond the minimum that one read instruction takes under the model."""
    total, minimum = 0, 0
    for first in range(0, 64, lanes_per_cycle):
        use = {}
        for a in addrs[first:first + lanes_per_cycle]:
            for b in range(0, nbytes, 4):
                bank = ((a + b) // 4) % 64
                use[bank] = use.get(bank, 0) + 1
        total += max(use.values())
        minimum += 1
    return total - minimum


def k_read(g, kb, t, c2):
    """Lane l reads 16 bytes of key 32 kb + l % 32, chunk 4 t + 2 (l / 32) + c2."""
    out = []
    for lane in range(64):
        key = 32 * kb + (lane & 31)
        out.append(key * D + ((4 * t + 2 * (lane >> 5) + c2) ^ g(key)) * 16)
    return out


def v_read(g, r, db):
    """Transposing read r of head-dim block db: lane pairs address one key, the even lane
    the first 8 bytes of the chunk, the odd lane the second."""
    out = []
    for lane in range(64):
        grp, j16 = lane >> 4, lane & 15
        e, par, hi = j16 >> 1, j16 & 1, lane >> 5
        key = 32 * (r >> 1) + 16 * (r & 1) + 8 * (e >> 2) + 4 * hi + (e & 3)
        out.append(key * D + ((2 * db + (grp & 1)) ^ g(key)) * 16 + 8 * par)
    return out


@pytest.mark.parametrize("g, k_extra, v_extra", [(g_old, 0, 2), (g_new, 0, 0)], ids=["old", "kernel"])
def test_bank_model_counts(g, k_extra, v_extra):
    for kb, t, c2 in itertools.product(range(2), range(2), range(2)):
        assert extra_cycles(k_read(g, kb, t, c2), 16, 16) == k_extra
    for r, db in itertools.product(range(4), range(4)):
        assert extra_cycles(v_read(g, r, db), 32, 8) == v_extra


def test_swizzle_is_a_row_permutation_shared_by_keys_16_apart():
    for k in range(64):
        assert sorted(c ^ g_new(k) for c in range(8)) == list(range(8))
        assert g_new(k) == g_new(k % 16)  # the V reads of a lane sit at fixed offsets
