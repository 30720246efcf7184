"""Helpers for the GPU parity tests: device marshalling and the comparison rules.

Index sets: the GPU must keep exactly N_eff = min(N, L_b) positions per query
head and match the oracle's set, except that positions whose oracle logit lies
within BAND of the oracle's N_eff-th largest logit t_N may be exchanged (the
GPU ranks fp32 logits, the oracle fp64 ones, so near-ties may order
differently). Outputs are then compared with the oracle evaluated on the
GPU's own set, so the output tolerance measures softmax and PV, not the
selection.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BAND = 1e-3            # near-threshold band, in scaled-logit units
TOL_BF16 = 2e-3        # max abs error of out for bf16 inputs (values ~ N(0,1))
TOL_F32 = 1e-5         # max abs error of out for fp32 inputs


def tol_for(dtype: str) -> float:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def to_device(x: dict) -> dict:
    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.cuda()
    return {"q": dev(x["q"]), "k": dev(x["k"]), "v": dev(x["v"]),
            "seq_lens": torch.from_numpy(np.ascontiguousarray(x["seq_lens"])).cuda()}


def rows_of(pairs, h_q):
    return [b * h_q + i for b, i in pairs]


def all_pairs(B, h_q):
    return [(b, i) for b in range(B) for i in range(h_q)]


def sample_pairs(B, h_q, n, seed=0):
    """n distinct (b, i) pairs spread over batch rows and heads (always includes corners)."""
    rng = np.random.default_rng(seed)
    chosen = {(0, 0), (B - 1, h_q - 1), (0, h_q - 1), (B - 1, 0)}
    while len(chosen) < min(n, B * h_q):
        chosen.add((int(rng.integers(B)), int(rng.integers(h_q))))
    return sorted(chosen)


def check_index_sets(gpu_idx: np.ndarray, ref: dict, x: dict, pairs, N: int):
    """gpu_idx [P][N] for the given pairs vs oracle result `ref` for the same pairs.

    Returns (number of rows whose set differs, total symmetric-difference size).
    """
    lens = x["seq_lens"]
    bad_rows = []
    for r, (b, i) in enumerate(pairs):
        n_eff = min(N, int(lens[b]))
        g = gpu_idx[r]
        assert (g[n_eff:] == -1).all(), f"pair {(b, i)}: slots past N_eff must be -1"
        gk = g[:n_eff]
        assert (gk >= 0).all() and (gk < lens[b]).all(), f"pair {(b, i)}: index out of range"
        assert (np.diff(gk) > 0).all(), f"pair {(b, i)}: kept indices must ascend strictly"
        if not np.array_equal(gk, ref["idx"][r, :n_eff]):
            bad_rows.append(r)
    diff_total = 0
    if bad_rows:
        sub = [pairs[r] for r in bad_rows]
        lg = oracle.logits(x["q"], x["k"], lens, pairs=sub)
        for j, r in enumerate(bad_rows):
            b, i = pairs[r]
            n_eff = min(N, int(lens[b]))
            sd = np.setxor1d(gpu_idx[r, :n_eff], ref["idx"][r, :n_eff])
            diff_total += len(sd)
            gap = np.abs(lg[j, sd] - ref["tN"][r])
            assert (gap <= BAND).all(), (
                f"pair {(b, i)}: positions {sd[gap > BAND][:8]} differ from the oracle set "
                f"by more than {BAND} from the threshold (gaps {gap[gap > BAND][:8]})")
    return len(bad_rows), diff_total


def check_outputs(gpu_out: np.ndarray, gpu_idx: np.ndarray, x: dict, pairs, tol: float):
    """gpu_out [P][d] vs the oracle's Eq. 7 on the GPU's own kept set."""
    ref_out, psum = oracle.attend_given(x["q"], x["k"], x["v"], x["seq_lens"], gpu_idx,
                                        pairs=pairs)
    err = np.abs(gpu_out.astype(np.float64) - ref_out)
    assert np.isfinite(gpu_out).all(), "non-finite output"
    assert err.max() <= tol, f"max abs error {err.max():.3e} > {tol:.1e}"
    return float(err.max())
