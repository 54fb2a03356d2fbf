"""Pins for the CPU oracle: hand-worked examples, closed forms, brute force,
library dense attention and invariants.  No GPU; nothing here reads the HIP
path."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dhsa_oracle as orc
from long_context_prefill_segmented_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_offsets(rng, L, lo, hi):
    o = [0]
    while o[-1] < L:
        o.append(min(L, o[-1] + int(rng.integers(lo, hi + 1))))
    return np.array(o, dtype=np.int64)


# ---------------------------------------------------------------- pooling


def test_pool_worked_example():
    g = _load("pool_worked_example.json")
    x = np.array(g["x"], dtype=np.float64)[:, None, :]
    got = orc.pool_chunks(x, g["offsets"])[0]
    np.testing.assert_allclose(got, np.array(g["expected"]), rtol=0, atol=1e-12)


def test_pool_constant_chunk_is_sqrt_n_times_value():
    rng = np.random.default_rng(0)
    offs = np.array([0, 1, 7, 64, 100])
    base = rng.standard_normal((4, 3, 5))
    x = np.repeat(base, np.diff(offs), axis=0)
    got = orc.pool_chunks(x, offs)
    for c, n in enumerate(np.diff(offs)):
        np.testing.assert_allclose(got[:, c], math.sqrt(n) * base[c], rtol=1e-13)


def test_pool_single_token_chunk_is_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 2, 4))
    got = orc.pool_chunks(x, np.arange(7))
    np.testing.assert_array_equal(got, np.transpose(x, (1, 0, 2)))


def test_pool_iid_unit_variance_for_any_length():
    # the length normalisation keeps pooled iid N(0,1) tokens at unit
    # variance whatever the chunk length (a plain mean gives 1/n, a sum n)
    rng = np.random.default_rng(2)
    for n in (4, 64, 400):
        C = 60
        offs = np.arange(C + 1) * n
        x = rng.standard_normal((C * n, 1, 128))
        p = orc.pool_chunks(x, offs)
        var = p.var()
        assert 0.9 < var < 1.1, (n, var)


def test_pool_linearity_and_prefix_form():
    rng = np.random.default_rng(3)
    offs = _rand_offsets(rng, 500, 1, 70)
    x = rng.standard_normal((500, 3, 8))
    y = rng.standard_normal((500, 3, 8))
    a, b = 1.5, -0.25
    lhs = orc.pool_chunks(a * x + b * y, offs)
    rhs = a * orc.pool_chunks(x, offs) + b * orc.pool_chunks(y, offs)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.pool_chunks_prefix(x, offs), orc.pool_chunks(x, offs),
                               rtol=1e-10, atol=1e-10)


def test_offsets_validation():
    with pytest.raises(ValueError):
        orc.check_offsets([0, 5, 5, 10], 10)
    with pytest.raises(ValueError):
        orc.check_offsets([1, 5, 10], 10)
    with pytest.raises(ValueError):
        orc.check_offsets([0, 5, 9], 10)
    orc.check_offsets([0, 10], 10)


# ---------------------------------------------------------------- scores


def test_scores_worked_example():
    g = _load("scores_worked_example.json")
    q = np.array(g["q"], dtype=np.float64)[:, None, :]
    k = np.array(g["k"], dtype=np.float64)[:, None, :]
    qb = orc.pool_chunks(q, g["offsets"])
    kb = orc.pool_chunks(k, g["offsets"])
    np.testing.assert_allclose(qb[0], np.array(g["qbar"]), atol=1e-14)
    np.testing.assert_allclose(kb[0], np.array(g["kbar"]), atol=1e-14)
    S = orc.chunk_scores(qb, kb)[0]
    for i, row in enumerate(g["scores_lower"]):
        np.testing.assert_allclose(S[i, :i + 1], row, atol=1e-14)
        assert np.all(np.isnan(S[i, i + 1:]))


def test_scores_unit_chunks_are_token_logits():
    # with every chunk one token long the chunk scores are the raw q.k logits
    rng = np.random.default_rng(4)
    L, Hq, Hkv, D = 12, 4, 2, 16
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    offs = np.arange(L + 1)
    S = orc.chunk_scores(orc.pool_chunks(q, offs), orc.pool_chunks(k, offs))
    for h in range(Hq):
        ref = torch.matmul(torch.from_numpy(q[:, h]), torch.from_numpy(k[:, h // 2]).T).numpy()
        np.testing.assert_allclose(np.tril(np.nan_to_num(S[h])), np.tril(ref), rtol=1e-12,
                                   atol=1e-12)


def test_scores_gqa_head_mapping():
    # query head h reads KV head h // (Hq/Hkv): heads 0,1 see the zero KV head
    C, D = 5, 8
    qb = np.ones((4, C, D))
    kb = np.stack([np.zeros((C, D)), np.ones((C, D))])
    S = orc.chunk_scores(qb, kb)
    low = np.tril(np.ones((C, C), dtype=bool))
    assert np.all(S[0][low] == 0) and np.all(S[1][low] == 0)
    assert np.all(S[2][low] == D) and np.all(S[3][low] == D)


def test_scores_gram_properties_when_q_equals_k():
    # Q = K: the diagonal is the squared norm and Cauchy-Schwarz bounds the rest
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 9, 6))
    S = orc.chunk_scores(x, x)[0]
    nrm2 = (x[0] ** 2).sum(axis=1)
    np.testing.assert_allclose(np.diag(S), nrm2, rtol=1e-14)
    for i in range(9):
        for j in range(i):
            assert abs(S[i, j]) <= math.sqrt(nrm2[i] * nrm2[j]) * (1 + 1e-14)


# ---------------------------------------------------------------- selection


def _parse(v):
    if v is None:
        return np.nan
    if isinstance(v, str):
        return float(v)
    return float(v)


def test_topk_worked_examples():
    g = _load("topk_worked_example.json")
    for case in g["cases"]:
        S = np.array([[_parse(v) for v in row] for row in case["scores"]], dtype=np.float64)
        got = [orc.select_row(S[i], i, case["k"]) for i in range(S.shape[0])]
        assert got == case["rows"], (case, got)


def _brute_force_row(s, i, k):
    # independent rank count: j < i is kept iff fewer than k-1 earlier chunks
    # beat it (higher score, or equal score and lower index)
    if i + 1 <= k:
        return list(range(i + 1))
    keep = []
    for j in range(i):
        better = 0
        for jj in range(i):
            if s[jj] > s[j] or (s[jj] == s[j] and jj < j):
                better += 1
        if better < k - 1:
            keep.append(j)
    return keep + [i]


def test_topk_vs_brute_force_with_ties():
    rng = np.random.default_rng(6)
    for trial in range(30):
        C = int(rng.integers(1, 40))
        k = int(rng.integers(1, 12))
        S = rng.integers(-3, 4, size=(C, C)).astype(np.float32)  # many ties
        S[S == 0] = np.where(rng.random((S == 0).sum()) < 0.5, -0.0, 0.0)
        for i in range(C):
            assert orc.select_row(S[i], i, k) == _brute_force_row(S[i], i, k)


def test_topk_invariants_and_full_budget():
    rng = np.random.default_rng(7)
    Hq, C = 3, 25
    S = rng.standard_normal((Hq, C, C)).astype(np.float32)
    for k in (1, 2, 5, 25, 40):
        rows = orc.select_topk(S, k)
        for h in range(Hq):
            for i in range(C):
                r = rows[h][i]
                assert r == sorted(r) and len(set(r)) == len(r)
                assert r[-1] == i                    # diagonal kept, last
                assert all(j <= i for j in r)        # no future chunk
                assert len(r) == min(k, i + 1)
                if k >= C:
                    assert r == list(range(i + 1))   # full causal chunk mask


def test_csr_round_trip():
    rng = np.random.default_rng(8)
    S = [rng.standard_normal((2, c, c)).astype(np.float32) for c in (7, 3)]
    rows = [orc.select_topk(s, 3) for s in S]
    rp, ci = orc.rows_to_csr(rows)
    assert rp[0] == 0 and rp[-1] == ci.size and len(rp) == 2 * 7 + 2 * 3 + 1
    assert orc.csr_to_rows(rp, ci, [7, 3], 2) == rows


# ---------------------------------------------------------------- attention


def test_attention_worked_example():
    g = _load("attention_worked_example.json")
    q = np.array([g["q"]])
    k = np.array(g["k"])
    v = np.array(g["v"])
    o, lse = orc.dense_masked_attention(q, k, v, np.ones((1, 2), dtype=bool), g["scale"])
    np.testing.assert_allclose(o[0], g["expected_out"], rtol=1e-13)
    np.testing.assert_allclose(lse[0], g["expected_lse"], rtol=1e-13)


def _sdpa_causal(q, k, v, scale):
    # library dense causal attention in float64 on the CPU; q [L,D]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=True, scale=scale)[0, 0].numpy()


def test_full_budget_equals_dense_causal_sdpa():
    rng = np.random.default_rng(9)
    L, Hq, Hkv, D = 200, 4, 2, 32
    offs = _rand_offsets(rng, L, 3, 30)
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    C = offs.size - 1
    _, _, _, _, rows = orc.build_mask(q, k, offs, C)   # k >= C keeps every causal chunk
    scale = 1.0 / math.sqrt(D)
    O, lse = orc.sparse_prefill(q, k, v, offs, rows, scale)
    for h in range(Hq):
        ref = _sdpa_causal(q[:, h], k[:, h // 2], v[:, h // 2], scale)
        np.testing.assert_allclose(O[:, h], ref, rtol=1e-11, atol=1e-12)
        z = scale * q[:, h] @ k[:, h // 2].T
        z[np.triu_indices(L, 1)] = -np.inf
        from scipy.special import logsumexp
        np.testing.assert_allclose(lse[h], logsumexp(z, axis=1), rtol=1e-12)


def test_budget_one_is_per_chunk_causal():
    rng = np.random.default_rng(10)
    L, D = 150, 16
    offs = _rand_offsets(rng, L, 5, 40)
    q = rng.standard_normal((L, 1, D))
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    _, _, _, _, rows = orc.build_mask(q, k, offs, 1)
    O, _ = orc.sparse_prefill(q, k, v, offs, rows, 0.3)
    for c in range(offs.size - 1):
        a, b = offs[c], offs[c + 1]
        ref = _sdpa_causal(q[a:b, 0], k[a:b, 0], v[a:b, 0], 0.3)
        np.testing.assert_allclose(O[a:b, 0], ref, rtol=1e-11, atol=1e-12)


def test_unit_chunks_budget_one_returns_v():
    rng = np.random.default_rng(11)
    L = 20
    q = rng.standard_normal((L, 2, 8))
    k = rng.standard_normal((L, 1, 8))
    v = rng.standard_normal((L, 1, 8))
    offs = np.arange(L + 1)
    _, _, _, _, rows = orc.build_mask(q, k, offs, 1)
    O, lse = orc.sparse_prefill(q, k, v, offs, rows)
    for h in range(2):
        np.testing.assert_allclose(O[:, h], v[:, 0], rtol=1e-14)
        np.testing.assert_allclose(lse[h], np.einsum("ld,ld->l", q[:, h], k[:, 0]) / math.sqrt(8),
                                   rtol=1e-12)


def test_constant_v_and_row_sums():
    rng = np.random.default_rng(12)
    L, D = 120, 16
    offs = _rand_offsets(rng, L, 4, 25)
    q = rng.standard_normal((L, 2, D)) * 3
    k = rng.standard_normal((L, 1, D)) * 3
    v = np.full((L, 1, D), 2.5)
    _, _, _, _, rows = orc.build_mask(q, k, offs, 3)
    O, _ = orc.sparse_prefill(q, k, v, offs, rows)
    np.testing.assert_allclose(O, 2.5, rtol=1e-13)
    # softmax rows sum to one: attention over v = one-hot columns
    v1 = np.zeros((L, 1, L))
    v1[np.arange(L), 0, np.arange(L)] = 1.0
    qq = np.concatenate([q, np.zeros((L, 2, L - D))], axis=2)
    kk = np.concatenate([k, np.zeros((L, 1, L - D))], axis=2)
    P, _ = orc.sparse_prefill(qq, kk, v1, offs, rows, scale=0.25)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, rtol=1e-12)
    assert np.all(P >= 0)


def test_gathered_form_equals_dense_masked_form():
    rng = np.random.default_rng(13)
    L, Hq, Hkv, D = 180, 2, 1, 16
    offs = _rand_offsets(rng, L, 2, 35)
    q = rng.standard_normal((L, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    _, _, _, _, rows = orc.build_mask(q, k, offs, 3)
    O, lse = orc.sparse_prefill(q, k, v, offs, rows, 0.2)
    for h in range(Hq):
        M = orc.token_mask(offs, rows[h])
        Od, ld = orc.dense_masked_attention(q[:, h], k[:, 0], v[:, 0], M, 0.2)
        np.testing.assert_allclose(O[:, h], Od, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[h], ld, rtol=1e-12)
        # the mask is causal and contains the diagonal
        assert not np.any(np.triu(M, 1)) and np.all(np.diag(M))


def test_empty_row_gives_zero_and_minus_inf():
    q = np.ones((3, 1, 4))
    k = np.ones((3, 1, 4))
    v = np.ones((3, 1, 4))
    offs = np.array([0, 2, 3])
    rows = [[[0], []]]
    O, lse = orc.sparse_prefill(q, k, v, offs, rows)
    assert np.all(O[2, 0] == 0) and lse[0, 2] == -np.inf


# ---------------------------------------------------------------- needles


def test_oracle_selects_planted_needles():
    w = synth.small_workload("needle_small", 1, 8192, 4, 2, (64, 192), "qkv_centroid",
                             topk=4, seed=21, needles=4)
    x = synth.generate(w)
    q = orc.widen_bf16(x.q[0])
    k = orc.widen_bf16(x.k[0])
    _, _, _, _, rows = orc.build_mask(q, k, x.offsets[0], x.topk)
    G = w.num_q_heads // w.num_kv_heads
    assert len(x.needles) == 4 * w.num_kv_heads
    for (_b, i, j, g) in x.needles:
        for h in range(g * G, (g + 1) * G):
            assert j in rows[h][i], (i, j, h)


# ---------------------------------------------------------------- budgets, recent window


def test_budget_recent_worked_example():
    g = _load("topk_budget_recent_worked_example.json")
    S = np.array([[_parse(v) for v in row] for row in g["scores"]], dtype=np.float64)
    got = [orc.select_row_ex(S[i], i, g["budgets"][i], g["recent"]) for i in range(S.shape[0])]
    assert got == g["rows"], got


def _brute_force_row_ex(s, i, budget, recent):
    # independent rank count over the older candidates, then the window
    if i + 1 <= budget + recent:
        return list(range(i + 1))
    older = i - recent
    keep = []
    for j in range(older):
        better = sum(1 for jj in range(older) if s[jj] > s[j] or (s[jj] == s[j] and jj < j))
        if better < budget - 1:
            keep.append(j)
    return keep + list(range(older, i + 1))


def test_budget_recent_vs_brute_force_and_closed_forms():
    rng = np.random.default_rng(14)
    for _ in range(25):
        C = int(rng.integers(1, 35))
        S = rng.integers(-3, 4, size=(C, C)).astype(np.float32)
        S[S == 0] = -0.0
        recent = int(rng.integers(0, 6))
        for i in range(C):
            budget = int(rng.integers(1, 8))
            got = orc.select_row_ex(S[i], i, budget, recent)
            assert got == _brute_force_row_ex(S[i], i, budget, recent)
            assert got[-1] == i and got == sorted(got) and len(got) == min(i + 1, budget + recent)
            # the recent window is always kept
            assert all(j in got for j in range(max(0, i - recent), i + 1))
            if budget == 1:
                assert got == list(range(max(0, i - recent), i + 1))
        # recent = 0 with a fixed budget is the plain fixed-budget selection
        k = int(rng.integers(1, 6))
        assert [orc.select_row_ex(S[i], i, k, 0) for i in range(C)] == \
            [_brute_force_row(S[i], i, k) for i in range(C)]


# ---------------------------------------------------------------- boundary NMS


def test_nms_worked_examples():
    g = _load("nms_worked_example.json")
    for case in g["cases"]:
        got = orc.nms_boundaries(np.array(case["p"]), case["min_gap"], case["threshold"])
        assert got.tolist() == case["offsets"], (case, got)


def _nms_recursive(p, g, tau):
    # independent formulation: keep the best candidate of the open interval,
    # cut out everything closer than g to it, recurse on both sides
    L = len(p)

    def rec(lo, hi):  # candidates in [lo, hi]
        best = None
        for t in range(max(lo, g), min(hi, L - g) + 1):
            if p[t] >= tau and (best is None or p[t] > p[best]):
                best = t
        if best is None:
            return []
        return rec(lo, best - g) + [best] + rec(best + g, hi)

    return [0] + rec(0, L) + [L]


def test_nms_vs_recursive_formulation_and_characterisation():
    rng = np.random.default_rng(21)
    for _ in range(300):
        L = int(rng.integers(1, 60))
        g = int(rng.integers(1, 8))
        tau = float(rng.choice([0.0, 0.3, 0.5, 0.8]))
        p = rng.integers(0, 6, size=L) / 5.0   # many exact ties
        got = orc.nms_boundaries(p, g, tau).tolist()
        assert got == _nms_recursive(p, g, tau), (p, g, tau)
        # well separated: every chunk holds >= g tokens (a one-chunk output
        # of a sequence shorter than g is the exception)
        assert got[0] == 0 and got[-1] == L
        if len(got) > 2:
            assert min(np.diff(got)) >= g
        # maximal: every candidate left out has a kept boundary closer than
        # g that ranks above it (or is an end of the sequence)
        kept = set(got)
        for t in range(L):
            if p[t] < tau or t in kept:
                continue
            blockers = [s for s in kept if abs(s - t) < g]
            assert any(s in (0, L) or p[s] > p[t] or (p[s] == p[t] and s < t) for s in blockers)


def test_nms_closed_forms():
    # min_gap 1: every candidate survives
    p = np.array([0.0, 0.6, 0.7, 0.1, 0.9, 0.5])
    assert orc.nms_boundaries(p, 1, 0.5).tolist() == [0, 1, 2, 4, 5, 6]
    # increasing ramp: boundaries every g tokens back from L - g
    L, g = 100, 7
    ramp = np.arange(L) / L
    want = [0] + list(range(L - g, g - 1, -g))[::-1] + [L]
    assert orc.nms_boundaries(ramp, g, 0.0).tolist() == want
    # isolated peaks farther apart than g are exactly the boundaries
    p = np.zeros(200)
    peaks = [20, 57, 90, 150]
    p[peaks] = 1.0
    assert orc.nms_boundaries(p, 16, 0.5).tolist() == [0] + peaks + [200]
    # NaN never becomes a boundary
    p[57] = np.nan
    assert orc.nms_boundaries(p, 16, 0.5).tolist() == [0, 20, 90, 150, 200]


def test_widen_bf16_matches_torch_on_every_bit_pattern():
    """bf16 -> float64 widening is exact: every one of the 65,536 bit
    patterns (signed zeros, subnormals, the largest finite values, infinities
    and NaNs) widens to the value torch's own bfloat16 -> float64 conversion
    gives."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.widen_bf16(bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # the sign of zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0x0000])
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    # smallest subnormal: 2^-133
    assert got[0x0001] == 2.0 ** -133
