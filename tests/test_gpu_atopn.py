"""GPU parity of the Atop-N entry points (stale threshold) against the fp64
CPU oracle.

Calibration must reproduce the exact top-N step bit for bit and give tau
within 1e-3 relative of the oracle's (logits agree to ~1e-5; tau = e^(T - LSE)
moves by at most e^(1e-3) - 1 when the N-th logit is within the 1e-3 tie band).
A stale step's kept set must contain every position whose oracle logit is at
least 1e-3 above the oracle's threshold theta = log(tau) + LSE and none more
than 1e-3 below it; when more than 2N positions reach the threshold, the kept
set is the first 2N of them. Outputs must be within 2e-3 (bf16) / 1e-5
(fp32) of the oracle's attention over the GPU's own kept set.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_helpers import all_pairs, to_device, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_asymmetric_gqa_amd as saga  # noqa: E402  (fails loudly if not built)

BAND = 1e-3


def _say(*a):
    print(*a, flush=True)


def _drift(q, seed, eps=0.2):
    """q + eps * N(0,1), in the storage dtype (a slowly moving query)."""
    rng = np.random.default_rng(seed)
    f = synth.as_f32(q) + np.float32(eps) * rng.standard_normal(q.shape).astype(np.float32)
    return f.astype(np.float32) if q.dtype == np.float32 else synth.f32_to_bf16_bits(f)


def _check_stale(x, dx, case, N, tau_rows, pairs, label, tau_dev=None):
    """One stale step on the GPU vs the oracle; tau_rows [P] are the thresholds of the pairs."""
    B, h_q, d = case.B, case.h_q, case.d
    cap = 2 * N
    if tau_dev is None:
        tau_all = np.full(B * h_q, np.nan, np.float32)
        for j, (b, i) in enumerate(pairs):
            tau_all[b * h_q + i] = tau_rows[j]
        tau_dev = torch.from_numpy(tau_all).cuda()
    idx = torch.empty((B, h_q, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, h_q), dtype=torch.int32, device="cuda")
    out = saga.atopn_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N, tau_dev, idx_out=idx,
                          count_out=cnt)
    torch.cuda.synchronize()
    rows = [b * h_q + i for b, i in pairs]
    g_idx = idx.reshape(-1, cap).cpu().numpy()[rows]
    g_cnt = cnt.reshape(-1).cpu().numpy()[rows]
    g_out = out.reshape(-1, d).cpu().numpy()[rows]
    tau64 = tau_dev.reshape(-1).cpu().numpy().astype(np.float64)[rows]
    ref = oracle.atopn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, tau64, pairs=pairs)
    z = oracle.logits(x["q"], x["k"], x["seq_lens"], pairs=pairs)
    nsat = 0
    for j, (b, i) in enumerate(pairs):
        L = int(x["seq_lens"][b])
        kept = g_idx[j][g_idx[j] >= 0]
        assert (g_idx[j][kept.size:] == -1).all(), label
        assert np.all(np.diff(kept) > 0), label
        th = ref["theta"][j]   # -inf for tau = 0 (every position), NaN for tau = NaN (none)
        if np.isnan(th) or L == 0:
            assert kept.size == 0 and g_cnt[j] == 0, label
            continue
        zr = z[j, :L]
        certain = np.nonzero(zr >= th + BAND)[0]
        possible = set(np.nonzero(zr >= th - BAND)[0].tolist())
        assert set(kept.tolist()) <= possible, (label, b, i)
        assert certain.size <= g_cnt[j] <= len(possible), (label, b, i, g_cnt[j])
        assert kept.size == min(int(g_cnt[j]), cap), (label, b, i)
        if g_cnt[j] > cap:
            nsat += 1
            last = kept[-1]
            assert set(certain[certain <= last].tolist()) <= set(kept.tolist()), (label, b, i)
        else:
            assert set(certain.tolist()) <= set(kept.tolist()), (label, b, i)
    # outputs: the oracle's Eq. 7 over the GPU's own kept set (zero when empty)
    sel = np.where(g_idx >= 0, g_idx, -1).astype(np.int32)
    exp_out, _ = oracle.attend_given(x["q"], x["k"], x["v"], x["seq_lens"], sel, pairs=pairs)
    err = float(np.abs(g_out - exp_out).max())
    assert err <= tol_for(case.dtype), (label, err)
    same = sum(set(g_idx[j][g_idx[j] >= 0].tolist()) == set(ref["idx"][j][ref["idx"][j] >= 0].tolist())
               for j in range(len(pairs)))
    _say(f"    {label}: rows={len(pairs)} same-set={same} saturated={nsat} "
         f"mean-count={g_cnt.mean():.1f} max|err|={err:.2e}")
    return g_cnt


SHAPES = [
    # (B, h_q, h_k, h_v, d, S_max, N, dtype, ragged)
    (2, 8, 2, 4, 64, 3000, 100, "bf16", True),
    (2, 8, 2, 4, 128, 2100, 64, "f32", True),
    (3, 12, 1, 2, 128, 5000, 300, "bf16", True),
    (2, 16, 1, 8, 64, 4100, 256, "bf16", False),
    (1, 6, 2, 3, 64, 777, 40, "bf16", False),       # a value head spanning two key heads
    (4, 12, 1, 2, 128, 32768, 1024, "bf16", True),  # 512-position K-scan items
]


@pytest.mark.parametrize("shape", SHAPES)
def test_calibration_is_the_exact_step_and_gives_the_oracle_tau(shape):
    B, h_q, h_k, h_v, d, S, N, dt, ragged = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=81)
    x = synth.make_inputs(case)
    dx = to_device(x)
    _say(f"[atopn] calibrate {shape}")
    i1 = torch.empty((B, h_q, N), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    out1, tau = saga.atopn_calibrate(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N, idx_out=i1)
    out2 = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(out1, out2)
    ref, _ = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], N)
    g = tau.reshape(-1).cpu().numpy().astype(np.float64)
    rel = np.abs(g - ref) / ref
    _say(f"    tau rel err max {rel.max():.2e}")
    assert rel.max() <= 1e-3


@pytest.mark.parametrize("shape", SHAPES)
def test_stale_steps_under_query_drift(shape):
    B, h_q, h_k, h_v, d, S, N, dt, ragged = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=82)
    x = synth.make_inputs(case)
    pairs = all_pairs(B, h_q)
    tau, _ = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], N)
    tau = tau.astype(np.float32)
    _say(f"[atopn] stale {shape}")
    # the calibration inputs themselves, then a drifting query, then looser /
    # tighter thresholds (the looser one saturates the 2N buffer in some rows)
    _check_stale(x, to_device(x), case, N, tau, pairs, "same q")
    xd = dict(x)
    xd["q"] = _drift(x["q"], seed=5)
    dxd = to_device(xd)
    for f in (1.0, 0.3, 0.05, 3.0):
        _check_stale(xd, dxd, case, N, tau * np.float32(f), pairs, f"drift, tau x {f}")


def test_threshold_edges_zero_nan_and_above_one():
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=2500, N=100, dtype="bf16",
                            seed=83)
    lens = np.array([2500, 150], np.int32)
    x = synth.make_inputs(case, lens)
    dx = to_device(x)
    pairs = all_pairs(2, 8)
    _say("[atopn] tau = 0 keeps every position up to 2N (dense recompute rows)")
    g = _check_stale(x, dx, case, 100, np.zeros(16, np.float32), pairs, "tau 0")
    assert list(g) == [2500] * 8 + [150] * 8
    _say("[atopn] tau = NaN and tau = 2 keep nothing: out = 0")
    for t in (np.nan, 2.0):
        tv = torch.full((2, 8), t, dtype=torch.float32, device="cuda")
        cnt = torch.empty((2, 8), dtype=torch.int32, device="cuda")
        out = saga.atopn_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 100, tv, count_out=cnt)
        torch.cuda.synchronize()
        assert not out.any() and not cnt.any()


def test_decode_loop_calibrating_every_few_steps():
    # one sequence batch decoding 6 tokens: the cache grows by a row per step
    # and the query drifts; calibration at steps 0 and 4, stale steps between
    case = synth.small_case(B=2, h_q=12, h_k=1, h_v=2, d=128, S_max=6000, N=256, dtype="bf16",
                            seed=84)
    lens0 = np.array([5990, 4000], np.int32)
    x = synth.make_inputs(case, lens0 + 6)
    dx = to_device(x)
    pairs = all_pairs(2, 12)
    q = x["q"]
    tau = None
    for step in range(6):
        lens = lens0 + step
        xs = dict(x)
        xs["q"] = q
        xs["seq_lens"] = lens
        dxs = dict(dx)
        dxs["q"] = to_device(xs)["q"]
        dxs["seq_lens"] = torch.from_numpy(lens).cuda()
        if step % 4 == 0:
            _say(f"[atopn] loop step {step}: calibrate")
            out, tau = saga.atopn_calibrate(dxs["q"], dxs["k"], dxs["v"], dxs["seq_lens"], 256)
            torch.cuda.synchronize()
            ref = oracle.topn_attn(xs["q"], xs["k"], xs["v"], lens, 256)
            err = np.abs(out.reshape(-1, 128).cpu().numpy() - ref["out"]).max()
            assert err <= tol_for("bf16")
        else:
            _check_stale(xs, dxs, case, 256, None, pairs, f"loop step {step}", tau_dev=tau)
        q = _drift(q, seed=100 + step, eps=0.1)


def test_headline_workload_stale_step():
    case = synth.CASES["qwen25_1p5b_b64_32k"]
    x = synth.make_inputs(case)
    dx = to_device(x)
    pairs = all_pairs(case.B, case.h_q)
    _say("[atopn] headline: calibrate on the GPU, then a stale step with a drifted query")
    _, tau = saga.atopn_calibrate(dx["q"], dx["k"], dx["v"], dx["seq_lens"], case.N)
    torch.cuda.synchronize()
    ref, _ = oracle.atopn_calibrate(x["q"], x["k"], x["seq_lens"], case.N, pairs=pairs)
    g = tau.reshape(-1).cpu().numpy()[[b * case.h_q + i for b, i in pairs]]
    assert (np.abs(g - ref) / ref).max() <= 1e-3
    xd = dict(x)
    xd["q"] = _drift(x["q"], seed=6, eps=0.1)
    dxd = dict(dx)
    dxd["q"] = to_device(xd)["q"]
    _check_stale(xd, dxd, case, case.N, None, pairs, "headline drift", tau_dev=tau)
