"""Pins of the key-merge oracle (oracle/merge.py) to facts the pages and the
mathematics fix, independent of the oracle's own formulas.

"More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding",
§4 (Eqs. 13-18, Lemma 4.1, Theorem 4.2), App. A (Eqs. 19-27), App. B
(Eqs. 28-35). Each test names the fact it checks.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

from oracle import merge as om
from synth.merge_inputs import MERGE_CASES, MergeCase, make_merge_inputs, planted_pairs


def _tiny(seed=5, L=60, D=24, h_q=4, h_kt=2, d=6):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((L, D)).astype(np.float32)
    Wq = (rng.standard_normal((h_q * d, D)) / math.sqrt(D)).astype(np.float32)
    Wk = (rng.standard_normal((h_kt * d, D)) / math.sqrt(D)).astype(np.float32)
    return X, Wq, Wk, h_q, h_kt, d


def test_trace_form_equals_frobenius_form():
    """App. A, Eqs. 20-23: the trace form equals the direct Eq. 13 sum of
    squared logit differences, for any M."""
    X, Wq, Wk, h_q, h_kt, d = _tiny()
    S = om.query_stats(X, Wq, h_q, h_kt, d)
    XtX = om.f64(X).T @ om.f64(X)
    rng = np.random.default_rng(1)
    for _ in range(3):
        M = rng.standard_normal((X.shape[1], d))
        direct = om.pair_loss_direct(X, Wq, Wk, h_q, h_kt, d, 0, 1, M)
        trace = om.pair_loss_trace(XtX, Wk, S, 0, 1, M, d)
        assert trace == pytest.approx(direct, rel=1e-10)


def test_closed_form_is_stationary_point_of_eq13():
    """Lemma 4.1: Eq. 15 minimises Eq. 13, so the loss has no first-order term
    there (central differences vanish) and rises in every direction."""
    X, Wq, Wk, h_q, h_kt, d = _tiny(seed=6)
    S = om.query_stats(X, Wq, h_q, h_kt, d)
    M = om.merged_projection(Wk, S, 0, 1, d)
    f0 = om.pair_loss_direct(X, Wq, Wk, h_q, h_kt, d, 0, 1, M)
    rng = np.random.default_rng(2)
    for _ in range(4):
        dM = rng.standard_normal(M.shape) * 1e-3
        fp = om.pair_loss_direct(X, Wq, Wk, h_q, h_kt, d, 0, 1, M + dM)
        fm = om.pair_loss_direct(X, Wq, Wk, h_q, h_kt, d, 0, 1, M - dM)
        curv = 0.5 * (fp + fm) - f0
        assert curv > 0
        assert abs(fp - fm) <= 1e-6 * curv + 1e-9 * f0


def test_normal_equations_hold():
    """Eq. 26: M (S_a + S_b) = W_K^a S_a + W_K^b S_b."""
    case = MERGE_CASES["merge_small"]
    inp = make_merge_inputs(case)
    S = om.query_stats(inp["x"], inp["wq"], case.h_q, case.h_kt, case.d)
    for a, b in itertools.combinations(range(case.h_kt), 2):
        M = om.merged_projection(inp["wk"], S, a, b, case.d)
        rhs = om.head_projection(inp["wk"], a, case.d) @ S[a] + \
            om.head_projection(inp["wk"], b, case.d) @ S[b]
        res = M @ (S[a] + S[b]) - rhs
        assert np.abs(res).max() <= 1e-9 * np.abs(rhs).max()


def test_identical_heads_merge_exactly():
    """W_K^a = W_K^b: the merged head is that head and w(a, b) = 0."""
    X, Wq, Wk, h_q, h_kt, d = _tiny(seed=7)
    Wk[d:] = Wk[:d]
    r = om.key_merge(X, Wq, Wk, h_q, h_kt, d)
    assert r["w"][0, 1] <= 1e-12 * np.trace(r["S"][0] @ r["S"][0])
    np.testing.assert_allclose(r["merged"][0], Wk[:d], atol=1e-10)


def test_equal_query_statistics_give_the_average():
    """S_a = S_b (the two query groups identical): Eq. 15 is the average of the
    two key projections, the merge App. B.1's baselines use."""
    X, Wq, Wk, h_q, h_kt, d = _tiny(seed=8)
    g = h_q // h_kt
    Wq[g * d:] = Wq[:g * d]
    r = om.key_merge(X, Wq, Wk, h_q, h_kt, d)
    avg = 0.5 * (Wk[:d].astype(np.float64) + Wk[d:].astype(np.float64))
    np.testing.assert_allclose(r["merged"][0], avg, atol=1e-10)


def test_rank_deficient_statistics():
    """Query projections with three dead output columns: S_a + S_b is
    singular, the pseudo-inverse (Penrose conditions) leaves those columns of
    the merge at zero, and the rest equals the merge of the problem without
    them."""
    X, Wq, Wk, h_q, h_kt, d = _tiny(seed=9, d=8)
    dead = [5, 6, 7]
    for j in range(h_q):
        Wq[j * d + np.array(dead)] = 0.0
    S = om.query_stats(X, Wq, h_q, h_kt, d)
    P = S[0] + S[1]
    Pp = om.pinv_psd(P, d)
    for lhs, rhs in ((P @ Pp @ P, P), (Pp @ P @ Pp, Pp), ((P @ Pp).T, P @ Pp),
                     ((Pp @ P).T, Pp @ P)):
        np.testing.assert_allclose(lhs, rhs, atol=1e-9 * np.abs(rhs).max())
    M = om.merged_projection(Wk, S, 0, 1, d)
    assert np.abs(M[:, dead]).max() == 0.0
    keep = [c for c in range(d) if c not in dead]
    sub = lambda W, h: np.concatenate([W[r * d + np.array(keep)] for r in range(h)])
    S2 = om.query_stats(X, sub(Wq, h_q), h_q, h_kt, len(keep))
    M2 = om.merged_projection(sub(Wk, h_kt), S2, 0, 1, len(keep))
    np.testing.assert_allclose(M[:, keep], M2, atol=1e-9 * np.abs(M2).max())


def test_pair_weight_bounds():
    """w(a, b) is the minimum of Eq. 13 (Eq. 16): 0 <= w <= the loss of the
    averaged merge and of M = 0."""
    case = MERGE_CASES["merge_small"]
    inp = make_merge_inputs(case)
    r = om.key_merge(inp["x"], inp["wq"], inp["wk"], case.h_q, case.h_kt, case.d)
    XtX = om.f64(inp["x"]).T @ om.f64(inp["x"])
    for a, b in itertools.combinations(range(case.h_kt), 2):
        avg = 0.5 * (om.head_projection(inp["wk"], a, case.d) +
                     om.head_projection(inp["wk"], b, case.d))
        l_avg = om.pair_loss_trace(XtX, inp["wk"], r["S"], a, b, avg, case.d)
        l_zero = om.pair_loss_trace(XtX, inp["wk"], r["S"], a, b, 0 * avg, case.d)
        assert 0.0 <= r["w"][a, b] <= l_avg
        assert r["w"][a, b] <= l_zero
    assert np.allclose(r["w"], r["w"].T) and np.all(np.diag(r["w"]) == 0)


def test_perfect_matching_count():
    """K_n (n even) has (n-1)!! perfect matchings, each pairing every head once."""
    for n in (2, 4, 6, 8, 10):
        ms = om.perfect_matchings(n)
        assert len(ms) == math.prod(range(n - 1, 0, -2))
        assert len({tuple(m) for m in ms}) == len(ms)
        for m in ms[:50]:
            assert sorted(h for p in m for h in p) == list(range(n))


def _dp_matching(w):
    """Minimum-weight perfect matching by dynamic programming over subsets
    (an algorithm independent of the oracle's enumeration)."""
    n = w.shape[0]
    best = {0: 0.0}
    for mask in range(1, 1 << n):
        if bin(mask).count("1") % 2:
            continue
        i = (mask & -mask).bit_length() - 1
        best[mask] = min(w[i, j] + best[mask ^ (1 << i) ^ (1 << j)]
                         for j in range(i + 1, n) if mask >> j & 1)
    return best[(1 << n) - 1]


def test_matching_against_subset_dp():
    """Theorem 4.2: the brute-force minimum equals the subset-DP minimum."""
    rng = np.random.default_rng(3)
    for n in (2, 4, 6, 8, 10):
        w = rng.random((n, n))
        w = w + w.T
        np.fill_diagonal(w, 0)
        pairs, tot = om.min_weight_matching(w)
        assert tot == pytest.approx(_dp_matching(w), rel=1e-12)
        assert sum(w[a, b] for a, b in pairs) == pytest.approx(tot, rel=1e-12)


def test_planted_pairing_is_recovered():
    """Heads built as near-duplicate pairs: the merge pairs them, and its total
    objective is below the other two initialisations of App. B.1."""
    case = MERGE_CASES["merge_small"]
    inp = make_merge_inputs(case)
    args = (inp["x"], inp["wq"], inp["wk"], case.h_q, case.h_kt, case.d)
    r = om.key_merge(*args)
    assert r["pairs"] == planted_pairs(case) != [(0, 1), (2, 3)]
    assert r["objective"] == pytest.approx(sum(r["w"][a, b] for a, b in r["pairs"]), rel=1e-12)
    rk = om.key_merge(*args, strategy="key")
    rs = om.key_merge(*args, strategy="sequential")
    assert r["objective"] <= rk["objective"] and r["objective"] < rs["objective"]


def test_relabelling_heads_relabels_the_result():
    """Renumbering the teacher key heads (with their query groups) permutes
    w accordingly and maps the matching onto the renumbered heads."""
    case = MergeCase("relabel", 300, 128, 8, 4, 16, seed=34)
    inp = make_merge_inputs(case)
    d, g = case.d, case.h_q // case.h_kt
    perm = [2, 0, 3, 1]   # new head i is old head perm[i]
    wk = np.concatenate([inp["wk"][p * d:(p + 1) * d] for p in perm])
    wq = np.concatenate([inp["wq"][(p * g) * d:(p * g + g) * d] for p in perm])
    r0 = om.key_merge(inp["x"], inp["wq"], inp["wk"], case.h_q, case.h_kt, d)
    r1 = om.key_merge(inp["x"], wq, wk, case.h_q, case.h_kt, d)
    np.testing.assert_allclose(r1["w"], r0["w"][np.ix_(perm, perm)], rtol=1e-9)
    mapped = sorted(tuple(sorted((perm[a], perm[b]))) for a, b in r1["pairs"])
    assert mapped == r0["pairs"]


def _gqa_module(x, wq, wk, wv, wo, h_q, h_k, d):
    """A plain GQA attention module without rotary embedding (fp64)."""
    T = x.shape[0]
    g = h_q // h_k
    q = (x @ om.f64(wq).T).reshape(T, h_q, d)
    k = (x @ om.f64(wk).T).reshape(T, h_k, d)
    v = (x @ om.f64(wv).T).reshape(T, h_k, d)
    heads = []
    for j in range(h_q):
        s = q[:, j] @ k[:, j // g].T / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        heads.append((p / p.sum(axis=1, keepdims=True)) @ v[:, j // g])
    return np.concatenate(heads, axis=1) @ om.f64(wo).T


def test_induced_permutations_leave_the_module_unchanged():
    """App. B: with key and value heads in sigma order and query heads / output
    blocks in pi_Q order the module computes the same function, and query
    head k of the permuted module uses teacher key head sigma[k // g]."""
    case = MergeCase("perm", 40, 64, 12, 4, 8, seed=34, dtype="f32")
    inp = make_merge_inputs(case, with_vo=True)
    g = case.h_q // case.h_kt
    sigma = [2, 0, 3, 1]
    pq = om.query_permutation(sigma, g)
    assert all(pq[k] // g == sigma[k // g] for k in range(case.h_q))
    wq, wv, wo = om.permute_heads(inp["wq"], inp["wv"], inp["wo"], sigma, case.h_q,
                                  case.h_kt, case.d)
    wk = np.concatenate([inp["wk"][r * case.d:(r + 1) * case.d] for r in sigma])
    x = om.f64(inp["x"])
    ref = _gqa_module(x, inp["wq"], inp["wk"], inp["wv"], inp["wo"], case.h_q, case.h_kt,
                      case.d)
    out = _gqa_module(x, wq, wk, wv, wo, case.h_q, case.h_kt, case.d)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_key_matching_weights():
    """Eq. 35: key-matching weights are the squared distance of realized keys,
    zero for identical heads and symmetric."""
    X, Wq, Wk, h_q, h_kt, d = _tiny(seed=10, h_q=8, h_kt=4)
    Wk[2 * d:3 * d] = Wk[0:d]
    w = om.key_weights(X, Wk, h_kt, d)
    assert w[0, 2] == 0.0 and w[1, 3] > 0 and np.allclose(w, w.T)
    pairs, _ = om.min_weight_matching(w)
    assert (0, 2) in pairs
