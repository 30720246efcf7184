"""GPU parity of the GQA -> SAGA key-head merge (saga_key_merge,
saga_merge_permute) against the fp64 oracle (oracle/merge.py).

"More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding",
§4 (Eqs. 13-17, Lemma 4.1, Theorem 4.2), App. A, App. B.

Tolerances, from the arithmetic: X^T X and the statistics accumulate bf16
products in fp32 over L tokens and D features, about 1e-6 relative to the
largest entry; the closed form and the pair weights inherit that error times
the conditioning of S_a + S_b (about 10 for these inputs):
  statistics   2e-5 x max |entry|
  pair weights 1e-4 x max weight
  merged keys  2e-4 x max |entry|
The matching must equal the oracle's where its best total beats every other
matching by more than 1e-3 relative, and otherwise be optimal for the
oracle's weights within that margin. The permutations are copies: bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import sparse_asymmetric_gqa_amd as saga
from oracle import merge as om
from synth.merge_inputs import MERGE_CASES, MergeCase, make_merge_inputs, planted_pairs

pytestmark = pytest.mark.gpu

TOL_STATS, TOL_W, TOL_M, GAP = 2e-5, 1e-4, 2e-4, 1e-3


def _dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _run(inp, case, strategy="logit"):
    print(f"[merge] {case.name} L={case.L} D={case.D} h_q={case.h_q} h_kt={case.h_kt} "
          f"d={case.d} {strategy}", flush=True)
    n, d = case.h_kt, case.d
    pw = torch.zeros((n, n), dtype=torch.float64, device="cuda")
    obj = torch.zeros((1,), dtype=torch.float64, device="cuda")
    stats = torch.zeros((n * d * d + (n * d) ** 2,), dtype=torch.float32, device="cuda")
    merged, sigma = saga.key_merge(_dev(inp["x"]), _dev(inp["wq"]), _dev(inp["wk"]), case.h_q,
                                   n, strategy, pair_w=pw, objective=obj, stats=stats)
    torch.cuda.synchronize()
    st = stats.cpu().numpy().astype(np.float64)
    return {"merged": merged.cpu().numpy().astype(np.float64), "sigma": sigma.cpu().tolist(),
            "w": pw.cpu().numpy(), "objective": float(obj.cpu()[0]),
            "S": st[:n * d * d].reshape(n, d, d), "H": st[n * d * d:].reshape(n * d, n * d)}


def _pairs(sigma):
    return [(sigma[2 * i], sigma[2 * i + 1]) for i in range(len(sigma) // 2)]


def _check_matching(gpu_pairs, ref_w):
    totals = sorted((sum(ref_w[a, b] for a, b in m), m) for m in om.perfect_matchings(ref_w.shape[0]))
    best = totals[0][0]
    gpu_total = sum(ref_w[a, b] for a, b in gpu_pairs)
    assert gpu_total <= best + GAP * max(abs(best), 1e-30)
    if len(totals) > 1 and totals[1][0] - best > GAP * max(abs(best), 1e-30):
        assert gpu_pairs == totals[0][1]
    for a, b in gpu_pairs:
        assert a < b
    assert [p[0] for p in gpu_pairs] == sorted(p[0] for p in gpu_pairs)


def _compare(g, r, case, strategy):
    n = case.h_kt
    assert np.abs(g["S"] - r["S"]).max() <= TOL_STATS * np.abs(r["S"]).max()
    assert np.abs(g["H"] - r["H"]).max() <= TOL_STATS * np.abs(r["H"]).max()
    if strategy != "sequential":
        wmax = np.abs(r["w"]).max()
        assert np.abs(g["w"] - r["w"]).max() <= TOL_W * wmax
        assert np.all(np.diag(g["w"]) == 0) and np.array_equal(g["w"], g["w"].T)
        _check_matching(_pairs(g["sigma"]), r["w"])
    else:
        assert g["sigma"] == list(range(n)) and not g["w"].any()
    assert sorted(g["sigma"]) == list(range(n))
    # merged keys: against the oracle's merge of the GPU's own pairs
    XtX = om.f64(case_inputs(case)["x"]).T @ om.f64(case_inputs(case)["x"])
    wk = case_inputs(case)["wk"]
    obj = 0.0
    for i, (a, b) in enumerate(_pairs(g["sigma"])):
        if strategy == "logit":
            M = om.merged_projection(wk, r["S"], a, b, case.d)
        else:
            M = 0.5 * (om.head_projection(wk, a, case.d) + om.head_projection(wk, b, case.d))
        obj += om.pair_loss_trace(XtX, wk, r["S"], a, b, M, case.d)
        ref = M.T
        assert np.abs(g["merged"][i] - ref).max() <= TOL_M * np.abs(ref).max(), (i, a, b)
    assert g["objective"] == pytest.approx(obj, rel=TOL_W)


_CACHE = {}


def case_inputs(case, with_vo=False):
    key = (case, with_vo)
    if key not in _CACHE:
        _CACHE[key] = make_merge_inputs(case, with_vo=with_vo)
    return _CACHE[key]


CASES = [
    MERGE_CASES["merge_small"],
    MergeCase("ragged_llama_like", 777, 400, 16, 8, 64, seed=42),    # L % 64, D % 256 ragged
    MergeCase("qwen_like_d128", 333, 512, 12, 2, 128, seed=46),
    MergeCase("d32_six_heads", 1000, 272, 12, 6, 32, seed=43),
    # splits of several 32-token stages (the load pipeline runs three stages
    # ahead), a last split with a partial stage, empty splits, and a ragged
    # feature block
    MergeCase("deep_ragged", 20001, 400, 8, 4, 64, seed=47),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("strategy", ["logit", "key", "sequential"])
def test_merge_matches_oracle(case, strategy):
    inp = case_inputs(case)
    r = om.key_merge(inp["x"], inp["wq"], inp["wk"], case.h_q, case.h_kt, case.d, strategy)
    g = _run(inp, case, strategy)
    _compare(g, r, case, strategy)
    if strategy == "logit" and case.h_kt > 2:
        assert _pairs(g["sigma"]) == planted_pairs(case)


def test_merge_identical_heads_and_dead_query_columns():
    """W_K^1 = W_K^0 merges to that head with weight 0; query heads with dead
    output columns give a singular S_a + S_b whose pseudo-inverse leaves those
    columns of the merge at 0 (exact zeros on both sides)."""
    case = MergeCase("degenerate", 500, 256, 8, 4, 64, seed=31)   # planted (0, 1), (2, 3)
    inp = dict(case_inputs(case))
    d = case.d
    wk = inp["wk"].copy()
    wk[d:2 * d] = wk[:d]
    wq = inp["wq"].copy()
    dead = np.array([3, 17, 60])
    for j in range(case.h_q):
        wq[j * d + dead] = 0
    inp.update(wk=wk, wq=wq)
    r = om.key_merge(inp["x"], wq, wk, case.h_q, case.h_kt, d)
    g = _run(inp, case)
    assert g["w"][0, 1] == 0.0
    assert _pairs(g["sigma"])[0] == (0, 1)
    keep = np.setdiff1d(np.arange(d), dead)
    np.testing.assert_allclose(g["merged"][0][keep], om.f64(wk[:d])[keep], rtol=0,
                               atol=TOL_M * 0.1)
    for i in range(case.h_kt // 2):
        assert not g["merged"][i][dead].any()
    XtX = om.f64(inp["x"]).T @ om.f64(inp["x"])
    for i, (a, b) in enumerate(_pairs(g["sigma"])):
        ref = om.merged_projection(wk, r["S"], a, b, d).T
        assert np.abs(g["merged"][i] - ref).max() <= TOL_M * np.abs(ref).max()
    assert g["objective"] == pytest.approx(
        sum(om.pair_loss_trace(XtX, wk, r["S"], a, b,
                               om.merged_projection(wk, r["S"], a, b, d), d)
            for a, b in _pairs(g["sigma"])), rel=TOL_W)


def test_merge_is_deterministic():
    case = MERGE_CASES["merge_small"]
    inp = case_inputs(case)
    g1, g2 = _run(inp, case), _run(inp, case)
    for k in ("merged", "w", "S", "H"):
        assert np.array_equal(g1[k], g2[k])
    assert g1["sigma"] == g2["sigma"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_permute_matches_oracle(dtype):
    case = MergeCase("perm", 64, 256, 12, 4, 32, seed=45, dtype=dtype)
    inp = case_inputs(case, with_vo=True)
    sigma = [2, 0, 3, 1]
    ref = om.permute_heads(inp["wq"], inp["wv"], inp["wo"], sigma, case.h_q, case.h_kt, case.d)
    out = saga.merge_permute(torch.tensor(sigma, dtype=torch.int32, device="cuda"),
                             _dev(inp["wq"]), _dev(inp["wv"]), _dev(inp["wo"]), case.h_q,
                             case.h_kt)
    torch.cuda.synchronize()
    for o, r in zip(out, ref):
        o = o.cpu()
        o = o.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else o.numpy()
        assert np.array_equal(o, r)


def test_merge_llama_layer_full_size():
    """The full Llama 3.2-1B layer (L = 128 Ki tokens, D 2048, 32 query heads,
    8 -> 4 key heads): S of key head 0 and the key-head-0 block of H against
    the oracle, the normal equations (Eq. 26) of every merge on the GPU's own
    statistics, the matching optimal for the GPU weights, and the planted
    pairing found."""
    case = MERGE_CASES["llama32_1b_layer"]
    inp = case_inputs(case)
    g = _run(inp, case)
    d, gq = case.d, case.h_q // case.h_kt
    Q = om.f64(inp["x"]) @ om.f64(inp["wq"][:gq * d]).T
    S0 = sum(Q[:, j * d:(j + 1) * d].T @ Q[:, j * d:(j + 1) * d] for j in range(gq))
    assert np.abs(g["S"][0] - S0).max() <= TOL_STATS * np.abs(S0).max()
    K0 = om.f64(inp["x"]) @ om.f64(inp["wk"][:d]).T
    H00 = K0.T @ K0
    assert np.abs(g["H"][:d, :d] - H00).max() <= TOL_STATS * np.abs(H00).max()
    for i, (a, b) in enumerate(_pairs(g["sigma"])):
        M = g["merged"][i].T
        P = g["S"][a] + g["S"][b]
        rhs = om.head_projection(inp["wk"], a, d) @ g["S"][a] + \
            om.head_projection(inp["wk"], b, d) @ g["S"][b]
        assert np.abs(M @ P - rhs).max() <= 1e-4 * np.abs(rhs).max()
    best = min(sum(g["w"][a, b] for a, b in m) for m in om.perfect_matchings(case.h_kt))
    assert sum(g["w"][a, b] for a, b in _pairs(g["sigma"])) == pytest.approx(best, rel=1e-12)
    assert _pairs(g["sigma"]) == planted_pairs(case)
    assert g["objective"] == pytest.approx(best, rel=1e-12)
    print(f"[merge] full-size pairs {_pairs(g['sigma'])} objective {best:.6e}", file=sys.stderr)
