"""Seeded synthetic inputs for the GQA -> SAGA key-head merge (input creation only).

Both the CPU oracle and the HIP path consume these arrays; this module holds
none of the merge arithmetic. The merge of "More Value per Key: Asymmetric
Sparse Attention for Faster LLM Decoding" (§4) runs on one attention module of
a trained GQA teacher and hidden states of a calibration set; neither is
available here, so:
  - X [L][D]: N(0,1) hidden states with a heavy-channel share (1% of the D
    features, at least one, scaled by 8), the large-magnitude channels that
    trained hidden states carry;
  - Wq [h_q*d][D], Wv [h_kt*d][D]: N(0, 1/D) entries; Wo [D][h_q*d]: N(0, 1/(h_q d));
  - Wk [h_kt*d][D]: teacher key heads in hidden pairs (a seeded permutation of
    the heads): both heads of a pair share an N(0, 1/D) base and add their
    own N(0, rho^2/D) part, so that a good pairing exists and is known.
Shapes are those of the two teachers the pages convert: Llama 3.2-1B
(D 2048, 32 query heads, 8 -> 4 key heads, d 64) and Qwen2.5-1.5B (D 1536,
12 query heads, 2 -> 1, d 128); L is a calibration sample of 128 sequences
of 1024 tokens (the pages do not give its size).
Storage: bf16 as uint16 bit patterns (or float32), C-contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import f32_to_bf16_bits, normal_tensor

STREAM_X, STREAM_WQ, STREAM_WK_BASE, STREAM_WK_OWN, STREAM_WV, STREAM_WO = 20, 21, 22, 23, 24, 25


@dataclass(frozen=True)
class MergeCase:
    name: str
    L: int
    D: int
    h_q: int
    h_kt: int
    d: int
    dtype: str = "bf16"
    seed: int = 11
    rho: float = 0.5


MERGE_CASES = {
    "merge_small": MergeCase("merge_small", 700, 512, 8, 4, 64, seed=34),
    "llama32_1b_layer": MergeCase("llama32_1b_layer", 131072, 2048, 32, 8, 64, seed=32),
    "qwen25_1p5b_layer": MergeCase("qwen25_1p5b_layer", 131072, 1536, 12, 2, 128, seed=33),
}


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    return a32 if dtype == "f32" else f32_to_bf16_bits(a32)


def planted_pairs(case: MergeCase) -> list:
    """The hidden pairing of Wk's heads, as sorted (a, b) pairs."""
    perm = np.random.default_rng(case.seed).permutation(case.h_kt)
    return sorted(tuple(sorted((int(perm[2 * i]), int(perm[2 * i + 1]))))
                  for i in range(case.h_kt // 2))


def heavy_channels(case: MergeCase) -> np.ndarray:
    n = max(1, case.D // 100)
    return np.random.default_rng(case.seed + 1).choice(case.D, size=n, replace=False)


def make_merge_inputs(case: MergeCase, with_vo: bool = False) -> dict:
    """X, Wq, Wk (and Wv, Wo when asked) for `case` (numpy, host memory)."""
    L, D, d, h_q, h_kt = case.L, case.D, case.d, case.h_q, case.h_kt
    x = normal_tensor(case.seed, STREAM_X, (L, D), "f32")
    x[:, heavy_channels(case)] *= 8.0
    sd = 1.0 / np.sqrt(D)
    wq = normal_tensor(case.seed, STREAM_WQ, (h_q * d, D), "f32") * sd
    base = normal_tensor(case.seed, STREAM_WK_BASE, (h_kt // 2, d, D), "f32") * sd
    own = normal_tensor(case.seed, STREAM_WK_OWN, (h_kt, d, D), "f32") * (case.rho * sd)
    wk = np.empty((h_kt, d, D), dtype=np.float32)
    for i, (a, b) in enumerate(planted_pairs(case)):
        wk[a] = base[i] + own[a]
        wk[b] = base[i] + own[b]
    out = {"x": _store(x, case.dtype), "wq": _store(wq, case.dtype),
           "wk": _store(wk.reshape(h_kt * d, D), case.dtype)}
    if with_vo:
        out["wv"] = _store(normal_tensor(case.seed, STREAM_WV, (h_kt * d, D), "f32") * sd,
                           case.dtype)
        out["wo"] = _store(normal_tensor(case.seed, STREAM_WO, (D, h_q * d), "f32")
                           / np.sqrt(h_q * d), case.dtype)
    return out
