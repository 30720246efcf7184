"""Pins for the oracle's Atop-N functions (stale threshold) against facts
fixed outside them.

"More Value per Key" §3.1 and App. C.1: a calibration step keeps the N-th
largest attention probability of each head as its threshold tau; later steps
keep the entries whose probability reaches tau (a logit threshold
log(tau) + LSE of the logits), at most 2N of them, and attend over those.
The pins tie the oracle to:
  - torch's float64 softmax and topk on logits computed by torch (an
    independent library path) for tau, and for which entries reach it;
  - closed forms: q = 0 (every probability is 1/L), a threshold no entry
    reaches (output 0), a threshold every entry reaches (the first 2N
    positions; full attention when 2N >= L, checked against torch SDPA);
  - invariants: the calibration step's own inputs give back its exact top-N
    set; a larger tau keeps a subset.
A slip such as comparing against the max logit instead of the log-sum-exp,
a strict/non-strict mix-up, a wrong cap or cap order fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _f64(a):
    return synth.as_f32(a).astype(np.float64)


def _torch_probs(x, b, i, h_q, h_k):
    """Softmax probabilities of row (b, i) over its L positions, in torch float64."""
    L = int(x["seq_lens"][b])
    d = x["q"].shape[-1]
    q = torch.from_numpy(_f64(x["q"][b, i]))
    k = torch.from_numpy(_f64(x["k"][b, i // (h_q // h_k), :L]))
    z = (k @ q) / np.sqrt(d)
    return torch.softmax(z, dim=0).numpy(), z.numpy()


SHAPES = [
    # (B, h_q, h_k, h_v, d, S_max, dtype, ragged, N)
    (2, 8, 2, 4, 64, 300, "bf16", True, 20),
    (1, 4, 1, 2, 64, 257, "f32", False, 64),
    (2, 12, 1, 2, 128, 180, "bf16", True, 40),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_calibration_tau_is_the_nth_largest_torch_probability(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged, N = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=71)
    x = synth.make_inputs(case)
    tau, lse = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], N)
    for r in range(B * h_q):
        b, i = divmod(r, h_q)
        p, z = _torch_probs(x, b, i, h_q, h_k)
        n = min(N, p.size)
        ref = torch.topk(torch.from_numpy(p), n).values[-1].item()
        assert tau[r] == pytest.approx(ref, rel=1e-12)
        assert lse[r] == pytest.approx(torch.logsumexp(torch.from_numpy(z), 0).item(), abs=1e-12)


def test_calibration_zero_query_gives_one_over_L():
    case = synth.small_case(B=2, h_q=4, h_k=1, h_v=2, d=64, S_max=97, N=10, dtype="bf16", seed=72)
    lens = np.array([97, 13], np.int32)
    x = synth.make_inputs(case, lens)
    x["q"][:] = 0
    for N in (1, 10, 200):
        tau, _ = oracle.atopn_calibrate(x["q"], x["k"], lens, N)
        for r in range(8):
            assert tau[r] == pytest.approx(1.0 / lens[r // 4], rel=1e-14)


@pytest.mark.parametrize("shape", SHAPES)
def test_stale_step_on_the_calibration_inputs_is_the_exact_topn(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged, N = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=73)
    x = synth.make_inputs(case)
    tau, _ = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], N)
    st = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, tau)
    ex = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N)
    for r in range(B * h_q):
        n = int(min(N, x["seq_lens"][r // h_q]))
        assert st["above"][r] == n
        assert list(st["idx"][r, :n]) == list(ex["idx"][r, :n])
        assert (st["idx"][r, n:] == -1).all()
    np.testing.assert_allclose(st["out"], ex["out"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
def test_kept_entries_are_exactly_those_whose_probability_reaches_tau(shape):
    B, h_q, h_k, h_v, d, S, dt, ragged, N = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=74)
    x = synth.make_inputs(case)
    rng = np.random.default_rng(5)
    probs = [_torch_probs(x, r // h_q, r % h_q, h_q, h_k)[0] for r in range(B * h_q)]
    # thresholds spread from below the smallest to above the N-th largest probability
    tau = np.array([np.exp(rng.uniform(np.log(p.min() * 0.5), np.log(np.sort(p)[-1] * 1.01)))
                    for p in probs])
    st = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, tau)
    for r, p in enumerate(probs):
        reach = np.nonzero(p >= tau[r])[0]
        assert st["above"][r] == reach.size
        kept = st["idx"][r][st["idx"][r] >= 0]
        assert list(kept) == list(reach[:2 * N])      # ascending, first 2N
        assert np.isclose(st["theta"][r], np.log(tau[r]) + np.log(np.sum(np.exp(
            _torch_probs(x, r // h_q, r % h_q, h_q, h_k)[1]))), atol=1e-9)


def test_threshold_reached_everywhere_keeps_the_first_2N_positions():
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=120, N=25, dtype="bf16",
                            seed=75)
    lens = np.array([120, 37], np.int32)
    x = synth.make_inputs(case, lens)
    tiny = np.full(16, 1e-300)
    st = oracle.atopn_attn(x["q"], x["k"], x["v"], lens, 25, tiny)
    for r in range(16):
        L = int(lens[r // 8])
        n = min(L, 50)
        assert st["above"][r] == L
        assert list(st["idx"][r, :n]) == list(range(n))
    # batch row 1 (L = 37 <= 2N): all positions kept, i.e. full attention (torch SDPA)
    q = torch.from_numpy(_f64(x["q"][1]))[:, None, :]
    k = torch.from_numpy(_f64(x["k"][1, :, :37])).repeat_interleave(4, dim=0)
    v = torch.from_numpy(_f64(x["v"][1, :, :37])).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, 0, :].numpy()
    np.testing.assert_allclose(st["out"][8:], ref, rtol=0, atol=1e-12)
    # batch row 0: the first 50 positions only
    g = oracle.attend_given(x["q"], x["k"], x["v"], lens,
                            np.tile(np.arange(50, dtype=np.int32), (8, 1)),
                            pairs=[(0, i) for i in range(8)])[0]
    np.testing.assert_allclose(st["out"][:8], g, rtol=0, atol=1e-12)


def test_zero_query_stale_step_is_the_mean_of_the_first_rows():
    case = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=90, N=30, dtype="f32", seed=76)
    x = synth.make_inputs(case)
    x["q"][:] = 0
    tau = np.full(4, 1.0 / 90)
    st = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 30, tau)
    v = _f64(x["v"])
    for i in range(4):
        assert st["above"][i] == 90
        np.testing.assert_allclose(st["out"][i], v[0, i // 2, :60].mean(axis=0), rtol=0, atol=1e-12)


def test_threshold_reached_nowhere_gives_zero():
    case = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=50, N=8, dtype="bf16", seed=77)
    x = synth.make_inputs(case)
    st = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 8, np.full(4, 2.0))
    assert (st["above"] == 0).all() and (st["idx"] == -1).all()
    assert not st["out"].any() and not st["psum"].any()


def test_larger_threshold_keeps_a_subset():
    case = synth.small_case(B=2, h_q=6, h_k=2, h_v=3, d=64, S_max=200, N=100, dtype="bf16",
                            seed=78)
    x = synth.make_inputs(case)
    tau, _ = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], 30)
    a = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 100, tau * 0.5)
    b = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 100, tau * 2.0)
    for r in range(12):
        sa = set(a["idx"][r][a["idx"][r] >= 0])
        sb = set(b["idx"][r][b["idx"][r] >= 0])
        assert sb <= sa and a["above"][r] >= b["above"][r]
        np.testing.assert_allclose(a["psum"][r], 1.0, atol=1e-12)
