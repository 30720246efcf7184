"""GPU parity of saga_sparq_attn (SparQ-style approximate scoring in front of
the top-N selector) against the fp64 CPU oracle.

Rules (the selection ranks fp32 approximate logits, the oracle fp64 ones):
  - dims: the GPU's r kept dims of each key head equal the oracle's, except
    where the r-th and (r+1)-th summed magnitudes are within 1e-5 (relative) of
    each other; such key heads only get the output checks below;
  - kept set: the window (last min(local, L) positions) exactly; of the rest,
    N - local positions, containing every position whose oracle approximate
    logit is more than 1e-3 above the oracle's last kept one, and none more
    than 1e-3 below it;
  - alpha within 1e-4 of the oracle's approximate softmax mass of the GPU's
    own kept set;
  - out within 2e-3 (bf16) / 1e-5 (fp32) of alpha y3 + (1 - alpha) v_mean,
    y3 the oracle's exact attention over the GPU's own kept set.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_helpers import BAND, all_pairs, to_device, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_asymmetric_gqa_amd as saga  # noqa: E402  (fails loudly if not built)


def _say(*a):
    print(*a, flush=True)


def _kt(x):
    """The S-contiguous copy of the keys: [B][h_k][d][S_max]."""
    return np.ascontiguousarray(np.swapaxes(x["k"], 2, 3))


def _vmean(x):
    v = synth.as_f32(x["v"]).astype(np.float64)
    out = np.zeros(v.shape[:2] + v.shape[3:], np.float32)
    for b, L in enumerate(x["seq_lens"]):
        if L > 0:
            out[b] = v[b, :, :L].mean(axis=1)
    return out


def _dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()


def _tied_groups(x, r):
    """Key heads whose r-th and (r+1)-th summed |q| are within 1e-5 (relative)."""
    q = synth.as_f32(x["q"]).astype(np.float64)
    B, h_q, d = q.shape
    h_k = x["k"].shape[1]
    g = h_q // h_k
    tied = set()
    if r >= d:
        return tied
    for b in range(B):
        for kh in range(h_k):
            u = np.sort(np.abs(q[b, kh * g:(kh + 1) * g]).sum(axis=0))[::-1]
            if u[r - 1] - u[r] <= 1e-5 * max(u[r - 1], 1e-30):
                tied.add((b, kh))
    return tied


def run_and_check(x, N, r, local, use_vmean, pairs, label, dtype):
    B, h_q, d = x["q"].shape
    h_k = x["k"].shape[1]
    g = h_q // h_k
    dx = to_device(x)
    kt = _dev(_kt(x))
    vm_np = _vmean(x) if use_vmean else None
    vm = _dev(vm_np) if use_vmean else None
    idx = torch.empty((B, h_q, N), dtype=torch.int32, device="cuda")
    alpha = torch.empty((B, h_q), dtype=torch.float32, device="cuda")
    dims = torch.empty((B, h_k, r), dtype=torch.int32, device="cuda")
    out = saga.sparq_attn(dx["q"], dx["k"], kt, dx["v"], dx["seq_lens"], N, r, local, v_mean=vm,
                          idx_out=idx, alpha_out=alpha, dims_out=dims)
    torch.cuda.synchronize()
    rows = [b * h_q + i for b, i in pairs]
    g_idx = idx.reshape(-1, N).cpu().numpy()[rows]
    g_alpha = alpha.reshape(-1).cpu().numpy()[rows]
    g_out = out.reshape(-1, d).cpu().numpy()[rows]
    g_dims = dims.cpu().numpy()
    ref = oracle.sparq_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, r, local,
                            vmean=None if vm_np is None else vm_np.astype(np.float64),
                            pairs=pairs, scores=True)
    tied = _tied_groups(x, r)
    lens = x["seq_lens"]
    exact_sets = 0
    for j, (b, i) in enumerate(pairs):
        L = int(lens[b])
        lw = min(local, L)
        Lp = L - lw
        ns = min(N - local, Lp)
        kept = g_idx[j][g_idx[j] >= 0]
        assert (g_idx[j][kept.size:] == -1).all(), (label, b, i)
        assert kept.size == ns + lw, (label, b, i, kept.size, ns + lw)
        assert np.all(np.diff(kept) > 0), (label, b, i)
        assert kept[ns:].tolist() == list(range(Lp, L)), (label, b, i)   # the window
        if (b, i // g) in tied:
            continue
        assert (g_dims[b, i // g] == ref["dims"][j]).all(), (label, b, i)
        zh = ref["zhat"][j]
        ranked = kept[:ns]
        if ns:
            th = ref["zthr"][j]
            assert (ranked < Lp).all()
            certain = set(np.nonzero(zh[:Lp] > th + BAND)[0].tolist())
            possible = set(np.nonzero(zh[:Lp] >= th - BAND)[0].tolist())
            rs = set(ranked.tolist())
            assert certain <= rs <= possible, (label, b, i)
            exact_sets += rs == set(ref["idx"][j][:ns].tolist())
        # alpha over the GPU's own set
        if L:
            m = zh[:L].max()
            lse = m + np.log(np.exp(zh[:L] - m).sum())
            a_ref = float(np.exp(zh[kept] - lse).sum())
            assert abs(g_alpha[j] - a_ref) <= 1e-4, (label, b, i, g_alpha[j], a_ref)
        else:
            assert g_alpha[j] == 0.0
    # outputs: exact attention over the GPU's own set, mixed with the GPU's alpha
    sel = np.where(g_idx >= 0, g_idx, -1).astype(np.int32)
    y3, _ = oracle.attend_given(x["q"], x["k"], x["v"], lens, sel, pairs=pairs)
    exp_out = y3.copy()
    if vm_np is not None:
        h_v = x["v"].shape[1]
        for j, (b, i) in enumerate(pairs):
            if int(lens[b]) > 0:
                a = float(g_alpha[j])
                exp_out[j] = a * y3[j] + (1 - a) * vm_np[b, i // (h_q // h_v)]
    err = float(np.abs(g_out - exp_out).max())
    assert err <= tol_for(dtype), (label, err)
    _say(f"    {label}: rows={len(pairs)} same-set={exact_sets} tied-groups={len(tied)} "
         f"alpha[min,max]=[{g_alpha.min():.3f},{g_alpha.max():.3f}] max|err|={err:.2e}")
    return g_idx, g_alpha, g_out


SHAPES = [
    # (B, h_q, h_k, h_v, d, S_max, N, r, local, dtype, ragged, vmean)
    (2, 8, 2, 4, 64, 3000, 100, 16, 25, "bf16", True, False),
    (2, 8, 2, 4, 128, 2104, 64, 32, 0, "f32", True, True),
    (3, 12, 1, 2, 128, 5000, 300, 32, 75, "bf16", True, True),
    (2, 16, 1, 8, 64, 4104, 256, 8, 64, "bf16", False, False),
    (1, 6, 2, 3, 64, 776, 40, 64, 10, "bf16", False, True),     # r = d
    (2, 4, 1, 2, 128, 1600, 50, 1, 5, "bf16", True, False),     # r = 1
    (2, 8, 2, 4, 64, 2000, 200, 24, 0, "f32", False, False),    # r not a multiple of 16
    (2, 12, 1, 2, 128, 3072, 1024, 48, 256, "bf16", False, True),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_sparq_small_shapes(shape):
    B, h_q, h_k, h_v, d, S, N, r, local, dt, ragged, vmean = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=101)
    x = synth.make_inputs(case)
    _say(f"[sparq] {shape}")
    run_and_check(x, N, r, local, vmean, all_pairs(B, h_q), str(shape), dt)


def test_sparq_edges_window_only_short_and_empty_rows():
    case = synth.small_case(B=4, h_q=8, h_k=2, h_v=4, d=64, S_max=2048, N=64, dtype="bf16",
                            seed=102)
    lens = np.array([0, 3, 40, 2048], np.int32)
    x = synth.make_inputs(case, lens)
    pairs = all_pairs(4, 8)
    _say("[sparq] window only (local = N)")
    g_idx, g_alpha, g_out = run_and_check(x, 64, 16, 64, True, pairs, "local=N", "bf16")
    assert not g_out[:8].any() and not g_alpha[:8].any()     # L = 0
    _say("[sparq] N >= L for the short rows: everything kept, alpha = 1")
    g_idx, g_alpha, _ = run_and_check(x, 64, 16, 16, True, pairs, "short rows", "bf16")
    assert np.allclose(g_alpha[8:24], 1.0, atol=1e-5)
    _say("[sparq] no window")
    run_and_check(x, 64, 32, 0, False, pairs, "local=0", "bf16")


def test_sparq_all_dims_no_window_is_the_exact_step():
    case = synth.small_case(B=2, h_q=12, h_k=1, h_v=2, d=128, S_max=4096, N=256, dtype="bf16",
                            ragged=True, seed=103)
    x = synth.make_inputs(case)
    pairs = all_pairs(2, 12)
    _say("[sparq] r = d, local = 0 against the exact path")
    g_idx, g_alpha, g_out = run_and_check(x, 256, 128, 0, False, pairs, "r=d", "bf16")
    dx = to_device(x)
    ex = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 256)
    torch.cuda.synchronize()
    assert np.abs(ex.reshape(-1, 128).cpu().numpy() - g_out).max() <= 2e-3


def test_sparq_clustered_rows_take_the_general_code():
    # the 300 best keys of batch row 0 crowd into its first chunk, so the
    # candidate lists cannot prove the ranked set exact; with r = d the
    # approximate logits are the exact ones
    case = synth.small_case(B=2, h_q=4, h_k=1, h_v=2, d=64, S_max=8192, N=320, dtype="bf16",
                            seed=104)
    x = synth.make_inputs(case)
    qsum = synth.as_f32(x["q"][0]).astype(np.float64).sum(axis=0)
    rng = np.random.default_rng(3)
    alpha = 3.0 * 2.0 ** (np.arange(300) / 60.0)
    rows = alpha[:, None] * qsum[None, :] / np.linalg.norm(qsum) * 8.0 + rng.standard_normal((300, 64))
    x["k"][0, 0, :300] = synth.f32_to_bf16_bits(rows.astype(np.float32))
    pairs = all_pairs(2, 4)
    for r, local in ((64, 20), (16, 20)):
        _say(f"[sparq] clustered, r={r} local={local}")
        g_idx, _, _ = run_and_check(x, 320, r, local, True, pairs, f"clustered r={r}", "bf16")
        if r == 64:
            assert set(g_idx[0][:300].tolist()) == set(range(300))


def test_sparq_deterministic_and_workspace_reuse():
    case = synth.small_case(B=3, h_q=12, h_k=1, h_v=2, d=128, S_max=6144, N=512, dtype="bf16",
                            ragged=True, seed=105)
    x = synth.make_inputs(case)
    dx = to_device(x)
    kt = _dev(_kt(x))
    ws = saga.new_workspace(saga.sparq_workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"],
                                                      512, 32), "cuda")
    outs = []
    for _ in range(3):
        outs.append(saga.sparq_attn(dx["q"], dx["k"], kt, dx["v"], dx["seq_lens"], 512, 32, 128,
                                    workspace=ws).clone())
        # an unrelated call in between reuses the same workspace with other sizes
        saga.sparq_attn(dx["q"], dx["k"], kt, dx["v"], dx["seq_lens"], 64, 8, 0, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_sparq_headline_shape():
    case = synth.CASES["qwen25_1p5b_b64_32k"]
    x = synth.make_inputs(case)
    pairs = all_pairs(case.B, case.h_q)
    for r, local in ((16, 256), (32, 256)):
        _say(f"[sparq] headline shape B=64 S=32K N=1024, r={r} local={local}")
        run_and_check(x, case.N, r, local, False, pairs, f"headline r={r}", "bf16")
