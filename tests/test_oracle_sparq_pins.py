"""Pins for the oracle's SparQ-style scorer (oracle.sparq_attn) against facts
fixed outside it.

"SparQ Attention: Bandwidth-Efficient LLM Inference", Steps 1-3 with the GQA
modifications: the r query dims with the largest summed magnitude over the
key head's query group; approximate scores over those dims with the
temperature sqrt(d * |q on dims|_1 / |q|_1); a local window of the last l
positions always kept, the rest of the budget by approximate score; exact
attention over the kept set; alpha = approximate softmax mass of the kept
set; out = alpha y3 + (1 - alpha) vmean when a running value mean is given.
The pins tie it to:
  - the exact top-N path (itself pinned) in the pages' two limits where the
    approximate scores are exact: r = d, and a query exactly sparse on r dims
    (temperature sqrt(d));
  - the pages' other temperature limit: equal magnitudes give sqrt(r);
  - torch (float64) for the dims (topk of summed magnitudes) and for alpha
    (softmax of the scores summed over the kept set);
  - the closed form of a zero query (uniform scores) with numpy means;
  - window edge cases and the linearity of Step 3 in vmean.
A slip such as summing |q| over the wrong group, sqrt of the wrong ratio,
dropping the window, selecting N instead of N - l, or mixing the scores of
the selection into the exact softmax fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _f64(a):
    return synth.as_f32(a).astype(np.float64)


def _bf16_or_f32(a, dt):
    a = np.asarray(a, np.float32)
    return a if dt == "f32" else synth.f32_to_bf16_bits(a)


def _torch_alpha(zhat_row, L, kept):
    p = torch.softmax(torch.from_numpy(zhat_row[:L]), dim=0)
    return float(p[torch.from_numpy(kept.astype(np.int64))].sum())


SHAPES = [
    # (B, h_q, h_k, h_v, d, S_max, dtype, ragged, N, r, l)
    (2, 8, 2, 4, 64, 300, "bf16", True, 40, 16, 10),
    (1, 4, 1, 2, 64, 257, "f32", False, 64, 8, 0),
    (2, 12, 1, 2, 128, 180, "bf16", True, 30, 32, 7),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_all_dims_without_window_is_the_exact_step(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged, N, _, _ = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=91)
    x = synth.make_inputs(case)
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, d, 0, scores=True)
    ex = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N)
    z = oracle.logits(x["q"], x["k"], x["seq_lens"])
    np.testing.assert_array_equal(sp["idx"], ex["idx"])
    np.testing.assert_allclose(sp["out"], ex["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sp["tau"], np.sqrt(d), rtol=1e-15)
    np.testing.assert_allclose(np.nan_to_num(sp["zhat"], nan=7.0), np.nan_to_num(z, nan=7.0),
                               rtol=0, atol=1e-12)
    assert (sp["dims"] == np.arange(d)).all()
    for r_ in range(B * h_q):
        L = int(x["seq_lens"][r_ // h_q])
        kept = sp["idx"][r_][sp["idx"][r_] >= 0]
        assert sp["alpha"][r_] == pytest.approx(_torch_alpha(z[r_], L, kept), abs=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
def test_exactly_sparse_group_query_scores_exactly(shape):
    """Every head of a key group is nonzero only on the same r dims: the
    approximate scores equal the exact logits (temperature sqrt(d)), so the
    kept set is the window plus the exact top N - l of the rest."""
    B, h_q, h_k, h_v, d, S, dt, ragged, N, r, l = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=92)
    x = synth.make_inputs(case)
    rng = np.random.default_rng(3)
    g = h_q // h_k
    q = _f64(x["q"]).astype(np.float32)
    supp = {}
    for b in range(B):
        for kh in range(h_k):
            s = np.sort(rng.choice(d, size=r, replace=False))
            supp[(b, kh)] = s
            mask = np.zeros(d, bool)
            mask[s] = True
            q[b, kh * g:(kh + 1) * g, ~mask] = 0.0
    x["q"] = _bf16_or_f32(q, dt)
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, r, l, scores=True)
    z = oracle.logits(x["q"], x["k"], x["seq_lens"])
    np.testing.assert_allclose(sp["tau"], np.sqrt(d), rtol=1e-15)
    lens = x["seq_lens"]
    for b in range(B):
        L = int(lens[b])
        lw = min(l, L)
        # the exact path on the prefix [0, L - l_eff) with budget N - l
        pre = dict(x)
        pre_lens = lens.copy()
        pre_lens[b] = L - lw
        ex = oracle.topn_attn(x["q"], x["k"], x["v"], pre_lens, max(N - l, 1),
                              pairs=[(b, i) for i in range(h_q)]) if N - l > 0 else None
        for i in range(h_q):
            j = b * h_q + i
            assert (sp["dims"][j] == supp[(b, i // g)]).all()
            np.testing.assert_allclose(sp["zhat"][j, :L], z[j, :L], rtol=0, atol=1e-12)
            kept = sp["idx"][j][sp["idx"][j] >= 0]
            want = list(range(L - lw, L))
            if ex is not None:
                ns = min(N - l, L - lw)
                want = sorted(ex["idx"][i][:ns].tolist()) + want
            assert kept.tolist() == want, (b, i)
            assert sp["alpha"][j] == pytest.approx(_torch_alpha(z[j], L, kept), abs=1e-12)
    given, _ = oracle.attend_given(x["q"], x["k"], x["v"], lens, sp["idx"])
    np.testing.assert_allclose(sp["out"], given, rtol=0, atol=1e-12)


def test_equal_magnitudes_give_temperature_sqrt_r():
    """|q[c]| constant within each head (random signs): the group sums tie on
    every dim, so the first r dims are kept and the temperature is sqrt(r)."""
    for dt, d, r in (("bf16", 64, 16), ("f32", 128, 32), ("bf16", 128, 1)):
        case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=d, S_max=100, N=20, dtype=dt,
                                seed=93)
        x = synth.make_inputs(case)
        rng = np.random.default_rng(4)
        mag = rng.choice([0.25, 0.5, 1.5, 3.0], size=(2, 8, 1))
        sgn = rng.choice([-1.0, 1.0], size=(2, 8, d))
        x["q"] = _bf16_or_f32(mag * sgn, dt)
        sp = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], 20, r, 5)
        assert (sp["dims"] == np.arange(r)).all()
        np.testing.assert_allclose(sp["tau"], np.sqrt(r), rtol=1e-15)


@pytest.mark.parametrize("shape", SHAPES)
def test_dims_are_torch_topk_of_group_magnitudes(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged, N, r, l = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=94)
    x = synth.make_inputs(case)
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, r, l)
    g = h_q // h_k
    q = torch.from_numpy(_f64(x["q"]))
    checked = 0
    for b in range(B):
        for kh in range(h_k):
            u = q[b, kh * g:(kh + 1) * g].abs().sum(0)
            vals, ind = torch.sort(u, descending=True, stable=True)
            if vals[r - 1] == vals[r] if r < d else False:
                continue   # a tie at the boundary: covered by the equal-magnitude pin
            want = np.sort(ind[:r].numpy())
            for i in range(kh * g, (kh + 1) * g):
                assert (sp["dims"][b * h_q + i] == want).all()
            checked += 1
    assert checked > 0


def test_zero_query_closed_form():
    """q = 0: every approximate score is 0 (uniform softmax 1/L), so the kept
    set is the first N - l positions plus the last l; the exact logits are 0
    too, so y3 is the plain mean of the kept value rows, alpha = N_eff / L, and
    with vmean = the mean of all L value rows out = alpha y3 + (1 - alpha) vmean."""
    case = synth.small_case(B=3, h_q=8, h_k=2, h_v=4, d=64, S_max=120, N=30, dtype="bf16",
                            seed=95)
    lens = np.array([120, 31, 9], np.int32)
    x = synth.make_inputs(case, lens)
    x["q"][:] = 0
    v = _f64(x["v"])
    vmean = np.stack([v[b, :, :max(int(lens[b]), 1)].mean(axis=1) for b in range(3)])
    for l in (0, 6, 30):
        sp = oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 30, 16, l, vmean=vmean)
        sp0 = oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 30, 16, l)
        for b in range(3):
            L = int(lens[b])
            lw = min(l, L)
            ns = min(30 - l, L - lw)
            want = list(range(ns)) + list(range(L - lw, L))
            for i in range(8):
                j = b * 8 + i
                assert (sp["dims"][j] == np.arange(16)).all() and sp["tau"][j] == 0.0
                kept = sp["idx"][j][sp["idx"][j] >= 0]
                assert kept.tolist() == want, (l, b, i)
                a = len(want) / L
                assert sp["alpha"][j] == pytest.approx(a, rel=1e-13)
                y3 = v[b, i // 2, want].mean(axis=0)
                np.testing.assert_allclose(sp0["out"][j], y3, rtol=0, atol=1e-12)
                np.testing.assert_allclose(sp["out"][j], a * y3 + (1 - a) * vmean[b, i // 2],
                                           rtol=0, atol=1e-12)


def test_window_edges():
    case = synth.small_case(B=2, h_q=4, h_k=1, h_v=2, d=64, S_max=80, N=16, dtype="f32",
                            seed=96)
    lens = np.array([80, 11], np.int32)
    x = synth.make_inputs(case, lens)
    # l = N: the last min(N, L) positions only
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 16, 8, 16)
    for j in range(8):
        L = int(lens[j // 4])
        kept = sp["idx"][j][sp["idx"][j] >= 0]
        assert kept.tolist() == list(range(max(L - 16, 0), L))
        assert np.isnan(sp["zthr"][j])
    # N >= L: everything is kept and alpha = 1 (full softmax mass)
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 100, 8, 20, vmean=np.ones((2, 2, 64)))
    full, _ = oracle.dense_attn(x["q"], x["k"], x["v"], lens)
    np.testing.assert_allclose(sp["alpha"], 1.0, atol=1e-13)
    np.testing.assert_allclose(sp["out"], full, rtol=0, atol=1e-12)
    # L = 0: nothing kept, out = 0, alpha = 0
    x0 = synth.make_inputs(case, np.array([0, 5], np.int32))
    sp = oracle.sparq_attn(x0["q"], x0["k"], x0["v"], x0["seq_lens"], 16, 8, 4,
                           vmean=np.ones((2, 2, 64)))
    assert (sp["idx"][:4] == -1).all() and not sp["out"][:4].any() and not sp["alpha"][:4].any()
    with pytest.raises(ValueError):
        oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 16, 65, 0)
    with pytest.raises(ValueError):
        oracle.sparq_attn(x["q"], x["k"], x["v"], lens, 16, 8, 17)


def test_selection_ranks_the_scored_prefix():
    """The non-window part of the kept set is a top-(N - l) set of the prefix
    by approximate score, equal scores broken by lower position."""
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=400, N=50, dtype="bf16",
                            ragged=True, seed=97)
    x = synth.make_inputs(case)
    sp = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], 50, 8, 12, scores=True)
    for j in range(16):
        L = int(x["seq_lens"][j // 8])
        lw = min(12, L)
        zh = sp["zhat"][j, :L - lw]
        kept = set(sp["idx"][j][(sp["idx"][j] >= 0) & (sp["idx"][j] < L - lw)].tolist())
        order = sorted(range(L - lw), key=lambda t: (-zh[t], t))
        assert kept == set(order[:min(38, L - lw)])


def test_mean_reallocation_is_affine_in_vmean():
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=200, N=24, dtype="bf16",
                            seed=98)
    x = synth.make_inputs(case)
    rng = np.random.default_rng(8)
    vm = rng.standard_normal((2, 4, 64))
    a = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], 24, 16, 6, vmean=vm)
    y3 = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], 24, 16, 6)
    for j in range(16):
        al = a["alpha"][j]
        assert 0.0 < al <= 1.0
        np.testing.assert_allclose(a["out"][j], al * y3["out"][j] + (1 - al) * vm[j // 8, (j % 8) // 2],
                                   rtol=0, atol=1e-12)
