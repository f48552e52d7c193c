"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: scalar brute
force, the page's online recurrence, closed forms, invariants, or library
special cases. Together they are chosen so that a dropped term, a wrong sign,
a wrong index or a transposed operand anywhere in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from workloads import make_decode, make_prefill, make_prefill_varlen

RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _tolist(a):
    return np.asarray(a).tolist()


# ---------------------------------------------------------------- brute force ----

@pytest.mark.parametrize("hq,hkv,nq,nk,d", [(1, 1, 1, 1, 1), (2, 2, 5, 5, 3), (4, 2, 7, 7, 4),
                                            (4, 1, 3, 9, 2), (2, 1, 9, 4, 4), (4, 4, 8, 8, 1)])
@pytest.mark.parametrize("causal,window,softcap", [(False, 0, 0.0), (True, 0, 0.0), (True, 3, 0.0),
                                                   (True, 1, 0.0), (False, 0, 2.5), (True, 2, 1.5),
                                                   (False, 4, 0.0)])
def test_brute_force_matches(hq, hkv, nq, nk, d, causal, window, softcap):
    q, k, v = _rand(hq, nq, d, scale=1.5), _rand(hkv, nk, d, scale=1.5), _rand(hkv, nk, d)
    scale = oracle.default_scale(d)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=scale, causal=causal, window=window, softcap=softcap)
    ob, lb = brute.brute_sdpa(_tolist(q), _tolist(k), _tolist(v), scale=scale, causal=causal,
                              window=window, softcap=softcap)
    ob, lb = np.array(ob), np.array(lb)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    fin = np.isfinite(lb)
    assert (np.isfinite(lse) == fin).all()
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def test_online_recurrence_equals_definition():
    for nk, d in [(1, 3), (6, 4), (17, 8)]:
        q, k, v = _rand(1, 1, d, scale=2.0), _rand(1, nk, d, scale=2.0), _rand(1, nk, d)
        scale = 1.0 / math.sqrt(d)
        o, _ = oracle.sdpa_fp64(q, k, v, scale=scale)
        row = brute.online_row(q[0, 0].tolist(), k[0].tolist(), v[0].tolist(), scale)
        np.testing.assert_allclose(o[0, 0], row, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms ----

def test_identical_keys_give_mean_of_values():
    n, d = 9, 4
    q = _rand(2, n, d)
    k = np.repeat(_rand(1, 1, d), n, axis=1).repeat(2, axis=0)
    v = _rand(2, n, d)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-12)
    oc, _ = oracle.sdpa_fp64(q, k, v, scale=0.3, causal=True)
    for i in range(n):
        np.testing.assert_allclose(oc[:, i], v[:, :i + 1].mean(axis=1), atol=1e-12)
    w = 3
    ow, _ = oracle.sdpa_fp64(q, k, v, scale=0.3, causal=True, window=w)
    for i in range(n):
        np.testing.assert_allclose(ow[:, i], v[:, max(0, i - w + 1):i + 1].mean(axis=1), atol=1e-12)


def test_dominant_score_selects_value_row():
    n, d = 12, 8
    for target in (0, 5, 11):
        q = np.zeros((1, 1, d)); q[0, 0, 0] = 10.0
        k = _rand(1, n, d, scale=0.01); k[0, :, 0] = 0.0; k[0, target, 0] = 4.0
        v = _rand(1, n, d)
        o, _ = oracle.sdpa_fp64(q, k, v, scale=1.0)  # gap >= 40 - 0.01*... in natural units
        np.testing.assert_allclose(o[0, 0], v[0, target], atol=n * math.exp(-39))


def test_probabilities_sum_to_one_and_masked_exactly_zero():
    q, k = _rand(2, 7, 4), _rand(1, 7, 4)
    for causal, window, cap in [(False, 0, 0.0), (True, 0, 0.0), (True, 3, 5.0)]:
        p = oracle.attention_probs(q, k, scale=0.5, causal=causal, window=window, softcap=cap)
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=2), 1.0, atol=1e-12)
        i, j = np.meshgrid(np.arange(7), np.arange(7), indexing="ij")
        masked = np.zeros((7, 7), bool)
        if causal:
            masked |= j > i
        if window:
            masked |= j <= i - window
        assert (p[:, masked] == 0.0).all()
        assert (p[:, ~masked] > 0.0).all()


def test_equal_scores_lse_is_log_count():
    n, d = 6, 3
    q = np.zeros((1, n, d)); k = _rand(1, n, d); v = _rand(1, n, d)
    _, lse = oracle.sdpa_fp64(q, k, v, scale=1.0)
    np.testing.assert_allclose(lse[0], math.log(n), atol=1e-12)
    _, lsec = oracle.sdpa_fp64(q, k, v, scale=1.0, causal=True)
    np.testing.assert_allclose(lsec[0], np.log(np.arange(1, n + 1)), atol=1e-12)


def test_single_key_and_head_dim_one():
    q, k, v = _rand(3, 1, 5), _rand(3, 1, 5), _rand(3, 1, 5)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.7)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse[:, 0], 0.7 * np.einsum("hd,hd->h", q[:, 0], k[:, 0]), atol=1e-12)
    # D = 1, two keys: weights form a logistic sigmoid of the score difference
    a, b0, b1, v0, v1 = 0.9, -1.3, 2.1, 3.0, -5.0
    o, lse = oracle.sdpa_fp64(np.array([[[a]]]), np.array([[[b0], [b1]]]),
                              np.array([[[v0], [v1]]]), scale=1.0)
    w1 = 1.0 / (1.0 + math.exp(a * b0 - a * b1))
    np.testing.assert_allclose(o[0, 0, 0], (1 - w1) * v0 + w1 * v1, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], math.log(math.exp(a * b0) + math.exp(a * b1)), atol=1e-13)


def test_golden_closed_forms():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
        o, lse = oracle.sdpa_fp64(q, k, v, scale=c["scale"], causal=c.get("causal", False))
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


# ---------------------------------------------------------------- invariants ----

def test_shift_invariance():
    n, d = 8, 4
    q, k, v = _rand(1, n, d), _rand(1, n, d), _rand(1, n, d)
    c = 0.75
    k[0, :, 2] = c
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.4, causal=True)
    q2 = q.copy(); q2[0, :, 2] += 1.9
    o2, lse2 = oracle.sdpa_fp64(q2, k, v, scale=0.4, causal=True)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 1.9 * c * 0.4, atol=1e-12)


def test_key_permutation_invariance():
    q, k, v = _rand(2, 5, 4), _rand(2, 11, 4), _rand(2, 11, 4)
    perm = RNG.permutation(11)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.5, softcap=3.0)
    o2, lse2 = oracle.sdpa_fp64(q, k[:, perm], v[:, perm], scale=0.5, softcap=3.0)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    q, k, v = _rand(8, 6, 4), _rand(2, 6, 4), _rand(2, 6, 4)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True)
    o2, lse2 = oracle.sdpa_fp64(q, np.repeat(k, 4, axis=0), np.repeat(v, 4, axis=0), scale=0.5,
                                causal=True)
    np.testing.assert_allclose(o, o2, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, atol=1e-15)
    # consecutive grouping: head h reads KV head h // 4, not h % 2
    o3, _ = oracle.sdpa_fp64(q, np.tile(k, (4, 1, 1)), np.tile(v, (4, 1, 1)), scale=0.5, causal=True)
    assert not np.allclose(o, o3)


def test_varlen_equals_concatenated_dense():
    case = make_prefill_varlen(lengths_q=[3, 7, 1, 5], num_q_heads=4, num_kv_heads=2, head_dim=8,
                               dtype="f32", seed=7, causal=True, window=3)
    q, k, v = (oracle.tensor_to_f64(t, "f32") for t in (case.q, case.k, case.v))
    cu = case.cu_seqlens_q
    o, lse = oracle.prefill_varlen(q, k, v, cu, cu, scale=0.35, causal=True, window=3)
    for b in range(4):
        a, z = cu[b], cu[b + 1]
        ob, lb = oracle.sdpa_fp64(q[a:z].transpose(1, 0, 2), k[a:z].transpose(1, 0, 2),
                                  v[a:z].transpose(1, 0, 2), scale=0.35, causal=True, window=3)
        np.testing.assert_allclose(o[a:z], ob.transpose(1, 0, 2), atol=1e-15)
        np.testing.assert_allclose(lse[:, a:z], lb, atol=1e-15)


def test_varlen_different_q_and_k_lengths_bottom_right():
    case = make_prefill_varlen(lengths_q=[2, 4], lengths_k=[6, 5], num_q_heads=2, num_kv_heads=1,
                               head_dim=4, dtype="f32", seed=8, causal=True)
    q, k, v = (oracle.tensor_to_f64(t, "f32") for t in (case.q, case.k, case.v))
    o, lse = oracle.prefill_varlen(q, k, v, case.cu_seqlens_q, case.cu_seqlens_k, scale=0.5)
    ob, lb = brute.brute_sdpa(_tolist(q[0:2].transpose(1, 0, 2)), _tolist(k[0:6].transpose(1, 0, 2)),
                              _tolist(v[0:6].transpose(1, 0, 2)), scale=0.5, causal=True)
    np.testing.assert_allclose(o[0:2], np.array(ob).transpose(1, 0, 2), atol=1e-12)
    np.testing.assert_allclose(lse[:, 0:2], np.array(lb), atol=1e-12)


def test_sampled_rows_equal_full_rows():
    case = make_prefill(batch=1, num_q_heads=2, num_kv_heads=1, seqlen_q=20, head_dim=4,
                        dtype="f32", seed=9, causal=True, window=5)
    q, k, v = (oracle.tensor_to_f64(t, "f32") for t in (case.q, case.k, case.v))
    o, lse = oracle.prefill_dense(q, k, v, scale=0.5, causal=True, window=5)
    rows = np.array([0, 4, 5, 19])
    o2, lse2 = oracle.prefill_dense(q, k, v, scale=0.5, causal=True, window=5, q_rows=rows,
                                    heads=np.array([1]))
    np.testing.assert_allclose(o2[:, 0], o[:, 1, rows], atol=0)
    np.testing.assert_allclose(lse2[:, 0], lse[:, 1, rows], atol=0)


def test_fully_masked_rows():
    # causal with Nq > Nk: the first Nq - Nk rows see no key
    q, k, v = _rand(1, 5, 3), _rand(1, 2, 3), _rand(1, 2, 3)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=1.0, causal=True)
    assert (o[0, :3] == 0).all() and np.isneginf(lse[0, :3]).all()
    assert np.isfinite(lse[0, 3:]).all()
    np.testing.assert_allclose(o[0, 3], v[0, 0], atol=1e-15)


def test_paged_equals_dense_decode_and_gather_is_exact():
    case = make_decode(lengths=[5, 33, 16, 1], num_q_heads=4, num_kv_heads=2, head_dim=8,
                       kv_dtype="bf16", seed=11, keep_logical=True)
    kc = oracle.tensor_to_f64(case.k_cache, "bf16")
    vc = oracle.tensor_to_f64(case.v_cache, "bf16")
    q = oracle.tensor_to_f64(case.q, "bf16")
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        g = oracle.gather_pages(kc, case.block_table[s], L)
        np.testing.assert_array_equal(g, oracle.tensor_to_f64(case.k_logical[s], "bf16"))
        assert not np.isnan(g).any()
    o, lse = oracle.decode_paged(q, kc, vc, case.block_table, case.seq_lens, scale=0.3)
    for s in range(case.num_seqs):
        kl = oracle.tensor_to_f64(case.k_logical[s], "bf16").transpose(1, 0, 2)
        vl = oracle.tensor_to_f64(case.v_logical[s], "bf16").transpose(1, 0, 2)
        ob, lb = brute.brute_sdpa(_tolist(q[s][:, None, :]), _tolist(kl), _tolist(vl), scale=0.3)
        np.testing.assert_allclose(o[s], np.array(ob)[:, 0], atol=1e-12)
        np.testing.assert_allclose(lse[s], np.array(lb)[:, 0], atol=1e-12)


def test_fp8_decode_uses_code_times_scale():
    case = make_decode(lengths=[20, 3], num_q_heads=2, num_kv_heads=2, head_dim=4,
                       kv_dtype="fp8_e4m3", seed=12, keep_logical=True)
    q = oracle.tensor_to_f64(case.q, "bf16")
    kc = oracle.tensor_to_f64(case.k_cache, "fp8_e4m3")
    vc = oracle.tensor_to_f64(case.v_cache, "fp8_e4m3")
    o, lse = oracle.decode_paged(q, kc, vc, case.block_table, case.seq_lens, scale=0.5,
                                 k_scale=case.k_scale, v_scale=case.v_scale)
    for s in range(2):
        kl = oracle.tensor_to_f64(case.k_logical[s], "fp8_e4m3") * case.k_scale[None, :, None]
        vl = oracle.tensor_to_f64(case.v_logical[s], "fp8_e4m3") * case.v_scale[None, :, None]
        ob, lb = brute.brute_sdpa(_tolist(q[s][:, None, :]), _tolist(kl.transpose(1, 0, 2)),
                                  _tolist(vl.transpose(1, 0, 2)), scale=0.5)
        np.testing.assert_allclose(o[s], np.array(ob)[:, 0], atol=1e-12)
        np.testing.assert_allclose(lse[s], np.array(lb)[:, 0], atol=1e-12)


def test_split_combine_associativity():
    q, k, v = _rand(3, 4, 6), _rand(3, 40, 6), _rand(3, 40, 6)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.6, softcap=4.0)
    bounds = [0, 7, 8, 23, 40]
    parts = [oracle.sdpa_fp64(q, k[:, a:b], v[:, a:b], scale=0.6, softcap=4.0)
             for a, b in zip(bounds[:-1], bounds[1:])]
    oc, lc = oracle.combine_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(lc, lse, atol=1e-12)
    # an empty range carries zero weight
    empty = oracle.sdpa_fp64(q, k[:, :0], v[:, :0], scale=0.6)
    oc2, lc2 = oracle.combine_partials(np.stack([empty[0]] + [p[0] for p in parts]),
                                       np.stack([empty[1]] + [p[1] for p in parts]))
    np.testing.assert_allclose(oc2, o, atol=1e-12)
    np.testing.assert_allclose(lc2, lse, atol=1e-12)


def test_softcap_limits():
    q, k, v = _rand(2, 6, 4, scale=3), _rand(2, 6, 4, scale=3), _rand(2, 6, 4)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True)
    o2, lse2 = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True, softcap=1e9)
    np.testing.assert_allclose(o2, o, atol=1e-9)
    np.testing.assert_allclose(lse2, lse, atol=1e-9)
    cap = 0.25
    _, lse3 = oracle.sdpa_fp64(q, k, v, scale=0.5, softcap=cap)
    assert (lse3 < cap + math.log(6)).all() and (lse3 > -cap + math.log(6)).all()


def test_window_limits():
    q, k, v = _rand(2, 9, 4), _rand(2, 9, 4), _rand(2, 9, 4)
    oc, lc = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True)
    ow, lw = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True, window=9)
    np.testing.assert_array_equal(ow, oc)
    o1, _ = oracle.sdpa_fp64(q, k, v, scale=0.5, causal=True, window=1)
    np.testing.assert_allclose(o1, v, atol=1e-15)
    # bottom-right alignment: with Nk = Nq + 3, W = 1 selects key i + 3
    k2, v2 = _rand(2, 12, 4), _rand(2, 12, 4)
    o2, _ = oracle.sdpa_fp64(q, k2, v2, scale=0.5, causal=True, window=1)
    np.testing.assert_allclose(o2, v2[:, 3:], atol=1e-15)


# ---------------------------------------------------------------- formats ----

def test_e4m3_table_matches_torch_float8_e4m3fn():
    table = oracle.e4m3_code_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(table) == nan).all()
    np.testing.assert_array_equal(table[~nan], ref[~nan])
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.nanmax(table) == 448.0 and table[1] == 2.0 ** -9


def test_widening_matches_torch():
    x = torch.from_numpy(RNG.standard_normal(4096).astype(np.float32) * 100)
    for name, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        t = x.to(dt)
        np.testing.assert_array_equal(oracle.tensor_to_f64(t, name), t.to(torch.float64).numpy())
    special = torch.tensor([0.0, -0.0, float("inf"), -float("inf"), 1e-40], dtype=torch.float32)
    t = special.to(torch.bfloat16)
    np.testing.assert_array_equal(oracle.tensor_to_f64(t, "bf16"), t.to(torch.float64).numpy())


def test_default_scale_is_binary32_rounding():
    for d in (32, 64, 128, 96):
        s = oracle.default_scale(d)
        assert s == float(np.float32(1 / math.sqrt(d)))
        assert abs(s - 1 / math.sqrt(d)) <= 2 ** -24 / math.sqrt(d)


# ------------------------------------------------------- chunked prefill over pages ----

def _paged_keys_by_loop(cache, row, L, page=16):
    """Token t of a sequence lives in slot t % page of physical page row[t // page];
    written with scalar indexing so it shares nothing with the oracle's gather."""
    out = []
    for t in range(L):
        p = int(row[t // page])
        out.append([[float(x) for x in cache[p, t % page, h]] for h in range(cache.shape[2])])
    # [L][Hkv][D] -> [Hkv][L][D]
    return [[out[t][h] for t in range(L)] for h in range(cache.shape[2])]


@pytest.mark.parametrize("causal,window,softcap", [(True, 0, 0.0), (False, 0, 0.0), (True, 5, 0.0),
                                                   (True, 0, 3.0)])
def test_paged_prefill_brute_force(causal, window, softcap):
    lens_k = [5, 33, 16, 1, 20]
    lens_q = [3, 17, 16, 1, 7]
    case = make_decode(lengths=lens_k, num_q_heads=4, num_kv_heads=2, head_dim=4,
                       kv_dtype="bf16", seed=21)
    kc = oracle.tensor_to_f64(case.k_cache, "bf16")
    vc = oracle.tensor_to_f64(case.v_cache, "bf16")
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    q = _rand(int(cu_q[-1]), 4, 4, scale=1.5)
    o, lse = oracle.prefill_paged(q, kc, vc, case.block_table, cu_q, case.seq_lens, scale=0.45,
                                  causal=causal, window=window, softcap=softcap)
    for b in range(len(lens_k)):
        a, z = int(cu_q[b]), int(cu_q[b + 1])
        kb = _paged_keys_by_loop(kc, case.block_table[b], lens_k[b])
        vb = _paged_keys_by_loop(vc, case.block_table[b], lens_k[b])
        ob, lb = brute.brute_sdpa(_tolist(q[a:z].transpose(1, 0, 2)), kb, vb, scale=0.45,
                                  causal=causal, window=window, softcap=softcap)
        np.testing.assert_allclose(o[a:z], np.array(ob).transpose(1, 0, 2), rtol=0, atol=1e-12)
        lb = np.array(lb)
        fin = np.isfinite(lb)
        assert (np.isfinite(lse[:, a:z]) == fin).all()
        np.testing.assert_allclose(lse[:, a:z][fin], lb[fin], rtol=0, atol=1e-12)


def test_paged_prefill_one_query_is_decode():
    # causal, one query per sequence: the query is the last position and sees every key
    lens = [7, 40, 16, 2]
    case = make_decode(lengths=lens, num_q_heads=4, num_kv_heads=1, head_dim=8,
                       kv_dtype="bf16", seed=22)
    kc = oracle.tensor_to_f64(case.k_cache, "bf16")
    vc = oracle.tensor_to_f64(case.v_cache, "bf16")
    q = oracle.tensor_to_f64(case.q, "bf16")              # [S, Hq, D]
    cu_q = np.arange(len(lens) + 1)
    o, lse = oracle.prefill_paged(q, kc, vc, case.block_table, cu_q, case.seq_lens, scale=0.3)
    od, ld = oracle.decode_paged(q, kc, vc, case.block_table, case.seq_lens, scale=0.3)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse.T, ld, rtol=0, atol=1e-13)


def test_paged_prefill_page_permutation_invariance():
    lens_k, lens_q = [33, 9], [33, 4]
    case = make_decode(lengths=lens_k, num_q_heads=2, num_kv_heads=2, head_dim=4,
                       kv_dtype="bf16", seed=23)
    kc = oracle.tensor_to_f64(case.k_cache, "bf16")
    vc = oracle.tensor_to_f64(case.v_cache, "bf16")
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    q = _rand(int(cu_q[-1]), 2, 4)
    o, lse = oracle.prefill_paged(q, kc, vc, case.block_table, cu_q, case.seq_lens, scale=0.5,
                                  window=7)
    perm = np.random.default_rng(3).permutation(kc.shape[0])
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[perm], vp[perm] = kc, vc                             # old page i is now page perm[i]
    bt = perm[case.block_table]
    o2, lse2 = oracle.prefill_paged(q, kp, vp, bt, cu_q, case.seq_lens, scale=0.5, window=7)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # and a block table that names a wrong page changes the answer
    bt_bad = case.block_table.copy()
    bt_bad[0, [0, 1]] = bt_bad[0, [1, 0]]
    o3, _ = oracle.prefill_paged(q, kc, vc, bt_bad, cu_q, case.seq_lens, scale=0.5, window=7)
    assert not np.allclose(o3[:33], o[:33])


def test_paged_prefill_sample_equals_full():
    case = make_decode(lengths=[40, 7, 19], num_q_heads=2, num_kv_heads=1, head_dim=4,
                       kv_dtype="bf16", seed=24)
    kc = oracle.tensor_to_f64(case.k_cache, "bf16")
    vc = oracle.tensor_to_f64(case.v_cache, "bf16")
    cu_q = np.array([0, 9, 16, 35])
    q = _rand(35, 2, 4)
    o, lse = oracle.prefill_paged(q, kc, vc, case.block_table, cu_q, case.seq_lens, scale=0.5)
    o2, lse2 = oracle.prefill_paged(q, kc, vc, case.block_table, cu_q, case.seq_lens, scale=0.5,
                                    seqs=[2], rows_per_seq={2: [0, 5, 18]}, heads=np.array([1]))
    rows = 16 + np.array([0, 5, 18])
    np.testing.assert_array_equal(o2[rows, 1], o[rows, 1])
    np.testing.assert_array_equal(lse2[1, rows], lse[1, rows])
    assert np.isnan(o2[:16]).all() and np.isnan(o2[rows, 0]).all()


# ------------------------------------------------------------------- attention sink ----

@pytest.mark.parametrize("hq,hkv,nq,nk,d", [(2, 1, 5, 5, 3), (4, 2, 7, 3, 4), (2, 2, 1, 9, 2)])
@pytest.mark.parametrize("causal,window,softcap", [(False, 0, 0.0), (True, 0, 0.0), (True, 2, 1.5)])
def test_sink_brute_force(hq, hkv, nq, nk, d, causal, window, softcap):
    q, k, v = _rand(hq, nq, d, scale=1.5), _rand(hkv, nk, d, scale=1.5), _rand(hkv, nk, d)
    sink = _rand(hq, scale=2.0)
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.6, causal=causal, window=window, softcap=softcap, sink=sink)
    ob, lb = brute.brute_sdpa(_tolist(q), _tolist(k), _tolist(v), scale=0.6, causal=causal, window=window,
                              softcap=softcap, sink=_tolist(sink))
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


def test_sink_closed_forms():
    # one key: O = v e^s / (e^s + e^sigma), LSE = ln(e^s + e^sigma)
    q, k, v = np.array([[[0.3, -1.2]]]), np.array([[[2.0, 0.5]]]), np.array([[[1.5, -4.0]]])
    s = (0.3 * 2.0 - 1.2 * 0.5) * 0.7
    sigma = 0.25
    o, lse = oracle.sdpa_fp64(q, k, v, scale=0.7, sink=np.array([sigma]))
    w = math.exp(s) / (math.exp(s) + math.exp(sigma))
    np.testing.assert_allclose(o[0, 0], [1.5 * w, -4.0 * w], rtol=1e-15)
    assert abs(lse[0, 0] - math.log(math.exp(s) + math.exp(sigma))) < 1e-15
    # a row with no allowed key: O = 0, LSE = sigma
    q5, k2, v2 = _rand(1, 5, 3), _rand(1, 2, 3), _rand(1, 2, 3)
    o, lse = oracle.sdpa_fp64(q5, k2, v2, scale=1.0, causal=True, sink=np.array([-0.5]))
    assert (o[0, :3] == 0).all() and (lse[0, :3] == -0.5).all()
    o, lse = oracle.sdpa_fp64(q5, k2[:, :0], v2[:, :0], scale=1.0, sink=np.array([1.25]))
    assert (o == 0).all() and (lse == 1.25).all()


def test_sink_rescales_the_sinkless_result():
    # from the definition: O_sink = O * e^LSE / (e^LSE + e^sigma), LSE_sink = logaddexp(LSE, sigma);
    # a sink far below every score changes nothing
    q, k, v = _rand(4, 6, 5), _rand(2, 11, 5), _rand(2, 11, 5)
    sink = np.array([0.0, 3.0, -2.0, 40.0])
    o0, l0 = oracle.sdpa_fp64(q, k, v, scale=0.45, causal=True, window=4)
    o1, l1 = oracle.sdpa_fp64(q, k, v, scale=0.45, causal=True, window=4, sink=sink)
    f = 1.0 / (1.0 + np.exp(sink[:, None] - l0))
    np.testing.assert_allclose(o1, o0 * f[..., None], rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(l1, np.logaddexp(l0, sink[:, None]), rtol=0, atol=1e-12)
    o2, l2 = oracle.sdpa_fp64(q, k, v, scale=0.45, causal=True, window=4, sink=np.full(4, -800.0))
    np.testing.assert_array_equal(o2, o0)
    np.testing.assert_array_equal(l2, l0)


def test_sink_passes_through_every_entry():
    sink = np.array([0.5, -1.0, 2.0, 0.0])
    case = make_decode(lengths=[5, 33], num_q_heads=4, num_kv_heads=2, head_dim=4, kv_dtype="bf16", seed=31,
                       keep_logical=True)
    kc, vc = (oracle.tensor_to_f64(t, "bf16") for t in (case.k_cache, case.v_cache))
    q = oracle.tensor_to_f64(case.q, "bf16")
    o, lse = oracle.decode_paged(q, kc, vc, case.block_table, case.seq_lens, scale=0.3, sink=sink)
    for s in range(2):
        kl = oracle.tensor_to_f64(case.k_logical[s], "bf16").transpose(1, 0, 2)
        vl = oracle.tensor_to_f64(case.v_logical[s], "bf16").transpose(1, 0, 2)
        ob, lb = brute.brute_sdpa(_tolist(q[s][:, None, :]), _tolist(kl), _tolist(vl), scale=0.3,
                                  sink=_tolist(sink))
        np.testing.assert_allclose(o[s], np.array(ob)[:, 0], atol=1e-12)
        np.testing.assert_allclose(lse[s], np.array(lb)[:, 0], atol=1e-12)
    # dense, sampled rows / heads, ragged and paged forms use the head's own sink
    qd, kd, vd = _rand(1, 4, 9, 3), _rand(1, 2, 9, 3), _rand(1, 2, 9, 3)
    o, lse = oracle.prefill_dense(qd, kd, vd, scale=0.5, causal=True, sink=sink)
    o2, lse2 = oracle.prefill_dense(qd, kd, vd, scale=0.5, causal=True, sink=sink, q_rows=np.array([2, 8]),
                                    heads=np.array([2]))
    np.testing.assert_array_equal(o2[0, 0], o[0, 2, [2, 8]])
    ob, lb = oracle.sdpa_fp64(qd[0], kd[0], vd[0], scale=0.5, causal=True, sink=sink)
    np.testing.assert_allclose(o[0], ob, atol=1e-15)
    cu = np.array([0, 9])
    ov, lv = oracle.prefill_varlen(qd[0].transpose(1, 0, 2), kd[0].transpose(1, 0, 2),
                                   vd[0].transpose(1, 0, 2), cu, cu, scale=0.5, causal=True, sink=sink)
    np.testing.assert_allclose(ov.transpose(1, 0, 2), ob, atol=1e-15)
    np.testing.assert_allclose(lv, lb, atol=1e-15)


# ------------------------------------------------------------------ fp8 prefill ----

def test_fp8_prefill_brute_force_on_decoded_codes():
    from workloads import make_prefill_fp8
    case = make_prefill_fp8(batch=1, num_q_heads=2, num_kv_heads=1, seqlen_q=5, seqlen_k=7, head_dim=4,
                            seed=41, causal=True)
    qc, kc, vc = (oracle.tensor_to_f64(t, "fp8_e4m3") for t in (case.q, case.k, case.v))
    o, lse = oracle.prefill_fp8(qc, kc, vc, q_scale=case.q_scale, k_scale=case.k_scale, v_scale=case.v_scale,
                                scale=0.5, causal=True)
    # decode the codes by the format's definition (sign, 4-bit exponent with bias 7, 3-bit mantissa)
    def dec(code):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        x = m * 2.0 ** -9 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        return -x if s else x
    bits = [t.view(torch.uint8).numpy() for t in (case.q, case.k, case.v)]
    qv = [[[dec(int(c)) * case.q_scale for c in row] for row in bits[0][0, h]] for h in range(2)]
    kv = [[[dec(int(c)) * case.k_scale for c in row] for row in bits[1][0, 0]]]
    vv = [[[dec(int(c)) * case.v_scale for c in row] for row in bits[2][0, 0]]]
    ob, lb = brute.brute_sdpa(qv, kv, vv, scale=0.5, causal=True)
    np.testing.assert_allclose(o[0], np.array(ob), rtol=0, atol=1e-12)
    fin = np.isfinite(np.array(lb))
    np.testing.assert_allclose(lse[0][fin], np.array(lb)[fin], rtol=0, atol=1e-12)


def test_fp8_prefill_scale_laws():
    q, k, v = np.round(_rand(1, 2, 6, 3) * 8), np.round(_rand(1, 2, 9, 3) * 8), np.round(_rand(1, 2, 9, 3) * 8)
    o1, l1 = oracle.prefill_fp8(q, k, v, q_scale=0.25, k_scale=0.5, v_scale=1.0, scale=0.3)
    # the value scale multiplies O and leaves the LSE; the product of the Q and K scales and the
    # softmax scale is all that reaches the scores
    o2, l2 = oracle.prefill_fp8(q, k, v, q_scale=0.25, k_scale=0.5, v_scale=3.0, scale=0.3)
    np.testing.assert_allclose(o2, 3.0 * o1, rtol=1e-14)
    np.testing.assert_array_equal(l2, l1)
    o3, l3 = oracle.prefill_fp8(q, k, v, q_scale=0.5, k_scale=1.0, v_scale=1.0, scale=0.075)
    np.testing.assert_allclose(o3, o1, rtol=1e-13)
    np.testing.assert_allclose(l3, l1, rtol=1e-13)


# ---------------------------------------------------------------------- backward ----

def _loss(q, k, v, do, **kw):
    o, _ = oracle.sdpa_fp64(q, k, v, **kw)
    return float((o * do).sum())


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(causal=True, window=3), dict(softcap=1.5),
                                dict(causal=True, sink=np.array([0.3, -1.0, 2.0, 0.0]))],
                         ids=["full", "causal", "window", "softcap", "sink"])
def test_backward_equals_finite_differences(kw):
    # L = sum(dO * O): its gradients are the backward's outputs
    q, k, v, do = _rand(4, 5, 3), _rand(2, 6, 3), _rand(2, 6, 3), _rand(4, 5, 3)
    kw = dict(kw, scale=0.7)
    dq, dk, dv = oracle.sdpa_backward_fp64(q, k, v, do, **kw)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = [xp if a is x else a for a in (q, k, v)]
            argm = [xm if a is x else a for a in (q, k, v)]
            num[idx] = (_loss(*args, do, **kw) - _loss(*argm, do, **kw)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)


def test_backward_matches_autograd_of_a_separate_forward():
    # torch float64 autograd through a forward written here (not the oracle's code)
    tq, tk, tv, tdo = (torch.from_numpy(x).requires_grad_(True) for x in
                       (_rand(4, 9, 5), _rand(2, 11, 5), _rand(2, 11, 5), _rand(4, 9, 5)))
    scale, cap = 0.45, 2.0
    kk, vv = tk.repeat_interleave(2, dim=0), tv.repeat_interleave(2, dim=0)
    s = cap * torch.tanh(scale * (tq @ kk.transpose(1, 2)) / cap)
    i = torch.arange(9)[:, None]
    j = torch.arange(11)[None, :]
    s = s.masked_fill(j > i + 2, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    (o * tdo).sum().backward()
    dq, dk, dv = oracle.sdpa_backward_fp64(tq.detach().numpy(), tk.detach().numpy(), tv.detach().numpy(),
                                           tdo.detach().numpy(), scale=scale, causal=True, softcap=cap)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_closed_forms():
    # one key: O = v exactly, so dV = sum of dO and dQ = dK = 0
    q, k, v, do = _rand(2, 3, 4), _rand(1, 1, 4), _rand(1, 1, 4), _rand(2, 3, 4)
    dq, dk, dv = oracle.sdpa_backward_fp64(q, k, v, do, scale=0.5)
    np.testing.assert_allclose(dv[0, 0], do.sum(axis=(0, 1)), atol=1e-14)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    # identical keys: uniform weights; dV_j = sum_i dO_i / Nk, dQ = 0
    k3 = np.tile(k, (1, 5, 1))
    dq, dk, dv = oracle.sdpa_backward_fp64(q, k3, _rand(1, 5, 4), do, scale=0.5)
    np.testing.assert_allclose(dv[0], np.tile(do.sum(axis=(0, 1)) / 5, (5, 1)), atol=1e-14)
    assert np.abs(dq).max() < 1e-13


# ------------------------------------------------- probabilities and batched backward ----

@pytest.mark.parametrize("hq,hkv,nq,nk,d", [(2, 1, 5, 7, 3), (4, 2, 6, 6, 4), (3, 3, 4, 9, 2)])
@pytest.mark.parametrize("causal,window,softcap", [(False, 0, 0.0), (True, 0, 0.0), (True, 2, 0.0),
                                                   (False, 0, 1.5), (True, 3, 2.0)])
def test_probabilities_equal_brute_force_weights(hq, hkv, nq, nk, d, causal, window, softcap):
    # With V the Nk x Nk identity, row i of O = P V is row i of P itself, so the scalar
    # brute force (math.fsum / math.exp loops) hands back the weight matrix entry by entry.
    q, k = _rand(hq, nq, d, scale=1.5), _rand(hkv, nk, d, scale=1.5)
    scale = oracle.default_scale(d)
    eye = [np.eye(nk).tolist() for _ in range(hkv)]
    ob, _ = brute.brute_sdpa(_tolist(q), _tolist(k), eye, scale=scale, causal=causal, window=window,
                             softcap=softcap)
    p = oracle.attention_probs(q, k, scale=scale, causal=causal, window=window, softcap=softcap)
    np.testing.assert_allclose(p, np.array(ob), rtol=0, atol=1e-13)
    # and P V is the definition's O for any V
    v = _rand(hkv, nk, 5)
    o, _ = oracle.sdpa_fp64(q, k, v, scale=scale, causal=causal, window=window, softcap=softcap)
    group = hq // hkv
    pv = np.stack([p[h] @ v[h // group] for h in range(hq)])
    np.testing.assert_allclose(pv, o, rtol=0, atol=1e-12)


def test_probabilities_of_two_keys_are_logistic():
    # two keys: P_0 = 1 / (1 + exp(s_1 - s_0)) with s_j = c tanh(scale q.k_j / c)
    q = np.array([[[1.0, 2.0]]])
    k = np.array([[[0.5, -1.0], [2.0, 1.5]]])
    for scale, cap in ((0.7, 0.0), (0.7, 1.25), (1.3, 0.5)):
        raw = np.array([1.0 * 0.5 + 2.0 * -1.0, 1.0 * 2.0 + 2.0 * 1.5]) * scale
        s = cap * np.tanh(raw / cap) if cap > 0 else raw
        p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        p = oracle.attention_probs(q, k, scale=scale, softcap=cap)
        np.testing.assert_allclose(p[0, 0], [p0, 1.0 - p0], rtol=0, atol=1e-15)


def test_batched_backward_equals_per_batch_and_finite_differences():
    # B = 2 with distinct inputs per batch entry, a sink and a causal mask: the batched
    # wrapper must hand each entry its own q, k, v and dO.
    b_, hq, hkv, n, d = 2, 4, 2, 5, 3
    q, k, v, do = _rand(b_, hq, n, d), _rand(b_, hkv, n, d), _rand(b_, hkv, n, d), _rand(b_, hq, n, d)
    sink = np.array([0.4, -0.8, 1.5, 0.0])
    kw = dict(scale=0.6, causal=True, sink=sink)
    dq, dk, dv = oracle.prefill_backward_dense(q, k, v, do, **kw)
    for b in range(b_):
        rq, rk, rv = oracle.sdpa_backward_fp64(q[b], k[b], v[b], do[b], **kw)
        np.testing.assert_allclose(dq[b], rq, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dk[b], rk, rtol=0, atol=1e-15)
        np.testing.assert_allclose(dv[b], rv, rtol=0, atol=1e-15)

    # central differences of sum(dO * O) through the batched forward (prefill_dense)
    def loss(qq, kk, vv):
        o, _ = oracle.prefill_dense(qq, kk, vv, scale=0.6, causal=True, sink=sink)
        return float((o * do).sum())

    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (loss(*[xp if a is x else a for a in (q, k, v)])
                        - loss(*[xm if a is x else a for a in (q, k, v)])) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7)
