"""Seeded synthetic inputs for SAGA decode attention (input creation only).

Both the CPU oracle and the HIP path consume these arrays; this module holds
none of the attention arithmetic. Shapes, value distributions and structure
follow the workloads the SAGA paper ("More Value per Key: Asymmetric Sparse
Attention for Faster LLM Decoding") measures on -- the attention shapes of
Llama 3.2-1B (8->4 key heads), Qwen2.5-1.5B (2->1) and SmolLM2-360M with
(h_k, h_v) = (1, 8) (§5.1, §5.2, App. C.2) -- with N(0,1) values and a 1%
share of heavy-hitter key rows standing in for trained caches, which are not
available here.

Layouts (all C-contiguous):
  q        [B][h_q][d]
  k_cache  [B][h_k][S_max][d]
  v_cache  [B][h_v][S_max][d]
  seq_lens int32 [B]
float32 tensors are numpy float32; bf16 tensors are numpy uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# sub-stream ids
STREAM_Q, STREAM_K, STREAM_V, STREAM_HEAVY, STREAM_LENS, STREAM_WINDOW = 0, 1, 2, 3, 4, 5


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_draws.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_fill_normal.argtypes = [u64, u64, i64, ctypes.c_int, vp, ctypes.c_int, vp]
        lib.synth_heavy_rows.argtypes = [u64, u64, ctypes.c_int, ctypes.c_int, i64, vp, vp,
                                         ctypes.c_double, vp]
        lib.synth_heavy_rows.restype = ctypes.c_int
        lib.synth_lengths.argtypes = [u64, u64, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


@dataclass(frozen=True)
class Case:
    """One workload: shapes, top-N size, storage dtype and generator recipe."""
    name: str
    B: int
    h_q: int
    h_k: int
    h_v: int
    d: int
    S_max: int
    N: int
    dtype: str            # "f32" or "bf16"
    seed: int
    heavy: str            # "fixed8" (8 rows per head) or "pct1" (floor(1% of L_b))
    heavy_factor: float
    ragged: bool = False  # lengths uniform in [S/2, S] per batch row
    # "uniform": heavy-hitter rows spread over all positions (the recipe above).
    # "recency_sink": attention concentrated the way trained models often
    # concentrate it -- on the first positions (sinks) and on a window of the
    # most recent ones -- on top of the uniform recipe (see _concentrate).
    structure: str = "uniform"

    def with_heads(self, h_k: int, h_v: int, seed: int | None = None) -> "Case":
        return replace(self, h_k=h_k, h_v=h_v, seed=self.seed if seed is None else seed)


# The five workloads. Seeds: config number; dense baselines use 100 + number.
CASES = {
    "tiny_fp32": Case("tiny_fp32", 1, 4, 1, 2, 64, 1024, 64, "f32", 1, "fixed8", 4.0),
    "llama32_1b_8to4": Case("llama32_1b_8to4", 8, 32, 4, 8, 64, 8192, 512, "bf16", 2, "pct1", 3.0),
    "qwen25_1p5b_2to1_ragged": Case("qwen25_1p5b_2to1_ragged", 16, 12, 1, 2, 128, 32768, 2048,
                                    "bf16", 3, "pct1", 3.0, ragged=True),
    "smollm2_360m_1x8": Case("smollm2_360m_1x8", 32, 16, 1, 8, 64, 16384, 1024, "bf16", 4,
                             "pct1", 3.0),
    "qwen25_1p5b_b64_32k": Case("qwen25_1p5b_b64_32k", 64, 12, 1, 2, 128, 32768, 1024, "bf16",
                                5, "pct1", 3.0),
}
CASE_ORDER = list(CASES)

# Concentrated-attention variants (not BASELINE configs): the same shapes with
# sink and recency structure, for the selector's worst case.
CONCENTRATED = {
    "qwen25_1p5b_b64_32k_recency": replace(CASES["qwen25_1p5b_b64_32k"],
                                           name="qwen25_1p5b_b64_32k_recency",
                                           structure="recency_sink"),
    "llama32_1b_8to4_recency": replace(CASES["llama32_1b_8to4"],
                                       name="llama32_1b_8to4_recency", structure="recency_sink"),
}
# sink positions, window length, and the logit gains aimed at (expected value
# for a window row at full strength, and for a sink row)
SINK_ROWS, WINDOW_ROWS = 4, 1024
WINDOW_GAIN, SINK_GAIN = 2.8, 5.0

# Dense (full-attention) baselines at the same shapes: (h_k, h_v) pairs.
DENSE_BASELINES = {
    "llama32_1b_8to4": [(8, 8)],
    "qwen25_1p5b_2to1_ragged": [(2, 2)],
    "smollm2_360m_1x8": [(8, 8), (4, 4)],
    "qwen25_1p5b_b64_32k": [(2, 2), (1, 2)],
}
SMOLLM_N_SWEEP = (512, 1024, 2048)


def lengths(case: Case) -> np.ndarray:
    lens = np.empty(case.B, dtype=np.int32)
    if case.ragged:
        _load().synth_lengths(case.seed, STREAM_LENS, case.B, case.S_max // 2, case.S_max,
                              _ptr(lens))
    else:
        lens[:] = case.S_max
    return lens


def _heavy_counts(case: Case, lens: np.ndarray) -> np.ndarray:
    if case.heavy == "fixed8":
        return np.minimum(lens, 8).astype(np.int32)
    if case.heavy == "pct1":
        return (lens.astype(np.int64) // 100).astype(np.int32)
    raise ValueError(case.heavy)


def normal_tensor(seed: int, stream: int, shape, dtype: str, row_scale=None) -> np.ndarray:
    """N(0,1) tensor of `shape` from stream (seed, stream); last axis is the row."""
    d = int(shape[-1])
    rows = int(np.prod(shape[:-1]))
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    if row_scale is not None:
        row_scale = np.ascontiguousarray(row_scale, dtype=np.float64).reshape(rows)
    _load().synth_fill_normal(seed, stream, rows, d, _ptr(row_scale),
                              0 if dtype == "f32" else 1, _ptr(out))
    return out


def make_inputs(case: Case, lens: np.ndarray | None = None) -> dict:
    """q, k_cache, v_cache and seq_lens for `case` (numpy, host memory)."""
    if lens is None:
        lens = lengths(case)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    B, S = case.B, case.S_max
    scale = np.ones((B, case.h_k, S), dtype=np.float64)
    rc = _load().synth_heavy_rows(case.seed, STREAM_HEAVY, B, case.h_k, S, _ptr(lens),
                                  _ptr(_heavy_counts(case, lens)), case.heavy_factor,
                                  _ptr(scale))
    if rc != 0:
        raise ValueError("bad lengths for heavy-row selection")
    q = normal_tensor(case.seed, STREAM_Q, (B, case.h_q, case.d), case.dtype)
    k = normal_tensor(case.seed, STREAM_K, (B, case.h_k, S, case.d), case.dtype, scale)
    v = normal_tensor(case.seed, STREAM_V, (B, case.h_v, S, case.d), case.dtype)
    if case.structure == "recency_sink":
        _concentrate(case, q, k, lens)
    elif case.structure != "uniform":
        raise ValueError(case.structure)
    return {"q": q, "k": k, "v": v, "seq_lens": lens, "heavy_scale": scale}


def _concentrate(case: Case, q: np.ndarray, k: np.ndarray, lens: np.ndarray) -> None:
    """Sink and recency structure, in place on k (input construction only).

    For every (b, key head) let u be the unit vector along the sum of the
    group's g = h_q / h_k query rows. The first SINK_ROWS positions get
    + a_s u and each position t of the last WINDOW_ROWS positions of the row
    gets + a_w r_t u, r_t uniform in [0.5, 1] from stream (seed, 5) at
    counter (b h_k + kh) 2^32 + t, with a = gain sqrt(g): a query row of the
    group has an expected component sqrt(d / g) along u, so a shift of a along
    u raises its scaled logit <q, K> / sqrt(d) by about a / sqrt(g) = gain
    (times r_t). Rows are modified in fp64 from their stored values and
    rounded back to the storage dtype.
    """
    B, h_q, d = q.shape
    h_k, S = k.shape[1], k.shape[2]
    g = h_q // h_k
    qf = as_f32(q).astype(np.float64)
    a_w = WINDOW_GAIN * np.sqrt(g)
    a_s = SINK_GAIN * np.sqrt(g)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        for kh in range(h_k):
            qs = qf[b, kh * g:(kh + 1) * g].sum(axis=0)
            u = qs / max(np.linalg.norm(qs), 1e-30)
            t0 = max(0, L - WINDOW_ROWS)
            draws = np.empty(L - t0, dtype=np.uint64)
            _load().synth_draws(case.seed, STREAM_WINDOW, ((b * h_k + kh) << 32) + t0, L - t0,
                                _ptr(draws))
            r = 0.5 + 0.5 * (draws >> np.uint64(11)).astype(np.float64) / float(1 << 53)
            gain = np.zeros(L)
            gain[t0:] = a_w * r
            ns = min(SINK_ROWS, L)
            gain[:ns] = np.maximum(gain[:ns], a_s)
            rows = np.nonzero(gain)[0]
            kr = as_f32(k[b, kh, rows]).astype(np.float64) + gain[rows, None] * u[None, :]
            k[b, kh, rows] = kr.astype(np.float32) if k.dtype == np.float32 else \
                f32_to_bf16_bits(kr.astype(np.float32))


def small_case(name="small", B=2, h_q=8, h_k=2, h_v=4, d=64, S_max=300, N=40, dtype="bf16",
               seed=7, heavy="pct1", heavy_factor=3.0, ragged=False) -> Case:
    """A workload small enough for exhaustive CPU checks."""
    return Case(name, B, h_q, h_k, h_v, d, S_max, N, dtype, seed, heavy, heavy_factor, ragged)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float32 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)
