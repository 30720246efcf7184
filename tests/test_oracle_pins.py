"""Pins for the CPU oracle against facts fixed outside it.

The oracle restates "More Value per Key: Asymmetric Sparse Attention for
Faster LLM Decoding" (Eq. 2 logits, Eq. 6 top-N, Eq. 7 softmax over the kept
entries, §3.2 SAGA head counts, App. B head blocks). These tests tie it to:
  - an independent library routine: torch's scaled_dot_product_attention in
    float64 on the CPU (N >= L reduces top-N attention to full attention);
  - brute force: the top-N set is the N-subset with the largest logit sum;
  - closed forms: q = 0 (uniform weights over the first N_eff positions),
    N = 1 (the argmax row), a single dominant key, equal value rows, a
    hand-built case with integer logits (tests/golden);
  - invariants: weights sum to 1, convex hull, value scaling, joint
    permutation of cache rows, SAGA == GQA on duplicated key heads.
Each is chosen so that a plausible slip (a dropped scale, a wrong head map, a
reversed tie rule, an off-by-one in N, reading rows past L) fails one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAN_BF16 = np.uint16(0x7FC0)


def _inputs(case, lens=None, nan_tail=True):
    x = synth.make_inputs(case, lens)
    if nan_tail:
        for b, L in enumerate(x["seq_lens"]):
            fill = np.float32(np.nan) if case.dtype == "f32" else NAN_BF16
            x["k"][b, :, L:, :] = fill
            x["v"][b, :, L:, :] = fill
    return x


def _f64(a):
    return synth.as_f32(a).astype(np.float64)


def _sdpa_full(x, h_q, h_k, h_v, mask=None):
    """Full attention via torch SDPA (float64, CPU), K/V expanded per query head."""
    q = torch.from_numpy(_f64(x["q"]))
    k = torch.from_numpy(_f64(x["k"])).repeat_interleave(h_q // h_k, dim=1)
    v = torch.from_numpy(_f64(x["v"])).repeat_interleave(h_q // h_v, dim=1)
    outs = []
    for b, L in enumerate(x["seq_lens"]):
        L = int(L)
        am = None if mask is None else torch.from_numpy(mask[b][:, None, :L])
        o = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :], k[b][:, :L], v[b][:, :L], attn_mask=am)
        outs.append(o[:, 0, :].numpy())
    return np.concatenate(outs, axis=0)


SHAPES = [
    # (B, h_q, h_k, h_v, d, S_max, dtype, ragged)
    (2, 8, 2, 4, 64, 200, "bf16", True),     # SAGA h_k < h_v, ragged
    (1, 4, 1, 2, 64, 130, "f32", False),     # tiny-config head layout
    (2, 6, 2, 2, 128, 90, "bf16", False),    # ordinary GQA h_k == h_v
    (3, 12, 1, 2, 128, 77, "bf16", True),    # Qwen-like head layout
    (2, 16, 1, 8, 64, 64, "f32", False),     # SmolLM-like (1, 8)
]


@pytest.mark.parametrize("shape", SHAPES)
def test_full_attention_limit_matches_sdpa(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=S, dtype=dt,
                            ragged=ragged, seed=11)
    x = _inputs(case)
    ref = _sdpa_full(x, h_q, h_k, h_v)
    for N in (int(x["seq_lens"].max()), S + 5):
        r = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N)
        np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)
    dense, _ = oracle.dense_attn(x["q"], x["k"], x["v"], x["seq_lens"])
    np.testing.assert_allclose(dense, ref, rtol=0, atol=1e-12)


def test_saga_equals_gqa_on_duplicated_key_heads():
    case = synth.small_case(B=2, h_q=16, h_k=2, h_v=8, d=64, S_max=150, N=20, ragged=True,
                            seed=5)
    x = _inputs(case, nan_tail=False)
    # K'[vh] = K[vh * h_k / h_v]: a GQA cache with h_kv = h_v whose key heads
    # repeat the SAGA key heads block-wise.
    src = (np.arange(8) * 2) // 8
    k_dup = np.ascontiguousarray(x["k"][:, src])
    a = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 20)
    b = oracle.topn_attn(x["q"], k_dup, x["v"], x["seq_lens"], 20)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
    # A wrong key-head map would pick other keys: check against a shuffled map.
    k_bad = np.ascontiguousarray(x["k"][:, ::-1])
    c = oracle.topn_attn(x["q"], k_bad, x["v"], x["seq_lens"], 20)
    assert not np.array_equal(a["idx"], c["idx"])


def test_bruteforce_subsets_tiny():
    rng = np.random.default_rng(3)
    B, h_q, h_k, h_v, d, S = 1, 4, 1, 2, 8, 9
    q = rng.standard_normal((B, h_q, d)).astype(np.float32)
    k = rng.standard_normal((B, h_k, S, d)).astype(np.float32)
    v = rng.standard_normal((B, h_v, S, d)).astype(np.float32)
    lens = np.array([S], np.int32)
    lg = np.einsum("bhd,bhsd->bhs", q.astype(np.float64),
                   np.repeat(k.astype(np.float64), h_q // h_k, axis=1)) / math.sqrt(d)
    for N in range(1, S + 1):
        r = oracle.topn_attn(q, k, v, lens, N)
        mask = np.zeros((B, h_q, S), dtype=bool)
        for i in range(h_q):
            best = max(itertools.combinations(range(S), N), key=lambda c: lg[0, i, list(c)].sum())
            assert list(r["idx"][i]) == list(best), (N, i)
            mask[0, i, list(best)] = True
        ref = _sdpa_full({"q": q, "k": k, "v": v, "seq_lens": lens}, h_q, h_k, h_v, mask=mask)
        np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-12)


def test_zero_query_selects_first_positions_uniformly():
    case = synth.small_case(B=3, h_q=8, h_k=2, h_v=4, d=64, S_max=120, N=50, seed=9)
    lens = np.array([120, 37, 1], np.int32)
    x = _inputs(case, lens)
    x["q"][:] = 0
    r = oracle.topn_attn(x["q"], x["k"], x["v"], lens, 50)
    v = _f64(x["v"])
    for j in range(3 * 8):
        b, i = divmod(j, 8)
        n = min(50, int(lens[b]))
        assert list(r["idx"][j, :n]) == list(range(n))
        assert (r["idx"][j, n:] == -1).all() and np.isneginf(r["sel"][j, n:]).all()
        np.testing.assert_allclose(r["out"][j], v[b, i // 2, :n].mean(axis=0), rtol=0,
                                   atol=1e-12)


def test_top1_is_argmax_and_lower_position_wins_ties():
    rng = np.random.default_rng(4)
    d, S = 32, 40
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, S, d)).astype(np.float32)
    v = rng.standard_normal((1, 2, S, d)).astype(np.float32)
    lens = np.array([S], np.int32)
    lg = (q[0].astype(np.float64) @ k[0, 0].astype(np.float64).T) / math.sqrt(d)
    r = oracle.topn_attn(q, k, v, lens, 1)
    for i in range(2):
        t = int(np.argmax(lg[i]))
        assert r["idx"][i, 0] == t
        np.testing.assert_array_equal(r["out"][i], v[0, i, t].astype(np.float64))
    # make rows 7 and 23 identical and dominant for head 0: the lower one wins
    k[0, 0, 7] = k[0, 0, 23] = 8.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    r = oracle.topn_attn(q, k, v, lens, 1)
    assert r["idx"][0, 0] == 7


def test_duplicate_row_straddling_threshold():
    case = synth.small_case(B=1, h_q=2, h_k=1, h_v=1, d=64, S_max=200, N=30, dtype="f32",
                            seed=21)
    x = _inputs(case, nan_tail=False)
    N = 30
    sc = oracle.logits(x["q"], x["k"], x["seq_lens"])[0]
    order = np.lexsort((np.arange(200), -sc))
    u = int(order[N - 1])                              # the N-th largest
    for w in (int(order[N + 5]), ):
        k2 = x["k"].copy()
        k2[0, 0, w] = k2[0, 0, u]                      # w now ties with u at rank N
        r = oracle.topn_attn(x["q"], k2, x["v"], x["seq_lens"], N)
        sel = set(r["idx"][0].tolist())
        assert min(u, w) in sel and max(u, w) not in sel
        assert set(order[:N - 1].tolist()) <= sel


def test_joint_permutation_of_cache_rows():
    case = synth.small_case(B=1, h_q=8, h_k=2, h_v=4, d=64, S_max=256, N=33, seed=13)
    x = _inputs(case, nan_tail=False)
    perm = np.random.default_rng(0).permutation(256)
    kp = np.ascontiguousarray(x["k"][:, :, perm])
    vp = np.ascontiguousarray(x["v"][:, :, perm])
    a = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 33)
    b = oracle.topn_attn(x["q"], kp, vp, x["seq_lens"], 33)
    for j in range(8):
        assert set(perm[b["idx"][j]].tolist()) == set(a["idx"][j].tolist())
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("N", [1, 7, 64, 500])
def test_weights_sum_to_one_and_convex_hull(N):
    case = synth.small_case(B=2, h_q=8, h_k=1, h_v=2, d=128, S_max=300, N=N, ragged=True,
                            seed=17)
    x = _inputs(case)
    r = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N)
    np.testing.assert_allclose(r["psum"], 1.0, rtol=0, atol=1e-12)
    v = _f64(x["v"])
    for j in range(16):
        b, i = divmod(j, 8)
        rows = v[b, i // 4, r["idx"][j][r["idx"][j] >= 0]]
        assert (r["out"][j] >= rows.min(axis=0) - 1e-12).all()
        assert (r["out"][j] <= rows.max(axis=0) + 1e-12).all()


def test_value_scaling_and_equal_rows():
    case = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=100, N=10, dtype="f32",
                            seed=23)
    x = _inputs(case, nan_tail=False)
    a = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 10)
    b = oracle.topn_attn(x["q"], x["k"], x["v"] * np.float32(4.0), x["seq_lens"], 10)
    np.testing.assert_allclose(b["out"], 4.0 * a["out"], rtol=0, atol=1e-12)
    assert (a["idx"] == b["idx"]).all()
    v_eq = np.broadcast_to(x["v"][:, :, :1], x["v"].shape).copy()
    c = oracle.topn_attn(x["q"], x["k"], v_eq, x["seq_lens"], 10)
    for j in range(4):
        np.testing.assert_allclose(c["out"][j], v_eq[0, j // 2, 0].astype(np.float64),
                                   rtol=0, atol=1e-12)


def test_single_dominant_key():
    case = synth.small_case(B=1, h_q=2, h_k=1, h_v=1, d=64, S_max=64, N=16, dtype="f32",
                            seed=29)
    x = _inputs(case, nan_tail=False)
    qv = x["q"][0, 0].astype(np.float64)
    x["k"][0, 0, 41] = (400.0 * qv / np.linalg.norm(qv)).astype(np.float32)
    r = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 16)
    np.testing.assert_allclose(r["out"][0], x["v"][0, 0, 41].astype(np.float64), rtol=0,
                               atol=1e-9)


def test_attend_given_and_logits_agree_with_topn():
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=180, N=25, ragged=True,
                            seed=31)
    x = _inputs(case)
    r = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 25)
    out, psum = oracle.attend_given(x["q"], x["k"], x["v"], x["seq_lens"], r["idx"])
    np.testing.assert_array_equal(out, r["out"])
    sc = oracle.logits(x["q"], x["k"], x["seq_lens"])
    for j in range(16):
        b = j // 8
        L = int(x["seq_lens"][b])
        assert np.isnan(sc[j, L:]).all()
        row = sc[j, :L]
        kept = r["idx"][j][r["idx"][j] >= 0]
        np.testing.assert_array_equal(row[kept], r["sel"][j, :len(kept)])
        assert row[kept].min() == r["tN"][j]
        assert (np.sort(row)[::-1][:25] == np.sort(row[kept])[::-1]).all()


def test_pairs_subset_matches_full_run():
    case = synth.small_case(B=3, h_q=4, h_k=1, h_v=2, d=64, S_max=90, N=12, seed=37)
    x = _inputs(case, nan_tail=False)
    full = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 12)
    pairs = [(2, 3), (0, 1), (1, 0)]
    sub = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 12, pairs=pairs)
    for r, (b, i) in enumerate(pairs):
        np.testing.assert_array_equal(sub["out"][r], full["out"][b * 4 + i])
        np.testing.assert_array_equal(sub["idx"][r], full["idx"][b * 4 + i])


def test_golden_integer_logit_cases():
    with open(os.path.join(GOLDEN, "integer_logits.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        d = c["d"]
        q = np.array(c["q"], np.float32).reshape(1, 1, d)
        k = np.array(c["k"], np.float32).reshape(1, 1, -1, d)
        v = np.array(c["v"], np.float32).reshape(1, 1, -1, d)
        lens = np.array([k.shape[2]], np.int32)
        r = oracle.topn_attn(q, k, v, lens, c["N"])
        n = len(c["expect_idx"])
        assert r["idx"][0, :n].tolist() == c["expect_idx"], c["name"]
        lg = np.array(c["expect_logits"], np.float64)
        w = np.exp(lg - lg.max())
        expect = (w / w.sum()) @ v[0, 0, c["expect_idx"]].astype(np.float64)
        np.testing.assert_allclose(r["out"][0], expect, rtol=0, atol=1e-15)
        np.testing.assert_allclose(r["sel"][0, :n], lg, rtol=0, atol=0)


def test_bad_arguments_are_rejected():
    q = np.zeros((1, 3, 8), np.float32)
    k = np.zeros((1, 2, 4, 8), np.float32)
    v = np.zeros((1, 3, 4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.topn_attn(q, k, v, np.array([4], np.int32), 2)   # 3 % 2 != 0
    q = np.zeros((1, 2, 8), np.float32)
    k = np.zeros((1, 1, 4, 8), np.float32)
    v = np.zeros((1, 2, 4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.attend_given(q, k, v, np.array([4], np.int32), np.array([[0, 4], [1, 2]]))


def test_concentrated_generator_crowds_the_top_n_into_the_recent_chunk():
    """The sink / recency variant of the generator (input construction only):
    on a reduced batch of each variant, the oracle's top-N sets put a large
    share of every head's kept positions in the last 1024 positions and keep
    the sink positions, which is the structure the variant stands for."""
    import synth
    for name in synth.CONCENTRATED:
        case = synth.replace(synth.CONCENTRATED[name], B=4)
        x = synth.make_inputs(case)
        r = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], case.N)
        share, sinks = [], []
        for j in range(case.B * case.h_q):
            L = int(x["seq_lens"][j // case.h_q])
            kept = r["idx"][j][r["idx"][j] >= 0]
            share.append(np.mean(kept >= L - synth.WINDOW_ROWS))
            sinks.append(np.sum(kept < synth.SINK_ROWS))
        assert np.median(share) >= 0.4, (name, np.median(share))
        assert np.mean(np.array(share) >= 0.3) >= 0.75, name
        assert np.mean(sinks) >= 3.0, name
        # the uniform recipe has no such structure
        u = synth.make_inputs(synth.replace(case, structure="uniform"))
        ru = oracle.topn_attn(u["q"], u["k"], u["v"], u["seq_lens"], case.N)
        L0 = int(u["seq_lens"][0])
        assert np.mean(ru["idx"][0] >= L0 - synth.WINDOW_ROWS) < 0.2
