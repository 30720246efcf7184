"""CPU oracle for SAGA top-N decode attention (fp64, plain C + OpenMP).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The product path never does.

The C source (oracle.c) restates "More Value per Key: Asymmetric Sparse
Attention for Faster LLM Decoding": Eq. 2 logits, Eq. 6 top-N selection,
Eq. 7 softmax over the kept entries and their value rows, §3.2 SAGA head
counts, App. B head blocks; the stale-threshold selector of §3.1 / App. C.1;
and "SparQ Attention: Bandwidth-Efficient LLM Inference" Steps 1-3 (with its
GQA modifications) as an approximate scorer in front of the same selector.
This wrapper only marshals numpy arrays.

Inputs: q [B][h_q][d], k [B][h_k][S_max][d], v [B][h_v][S_max][d] as float32
or as uint16 bf16 bit patterns; seq_lens int32 [B].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_topn_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i64, i, i, vp, i64,
                                         vp, vp, vp, vp, vp, i]
        lib.oracle_dense_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i64, i, vp, i64, vp, i]
        lib.oracle_logits.argtypes = [vp, vp, vp, i, i, i, i, i64, i, vp, i64, vp, i]
        lib.oracle_attend_given.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i64, i, i, vp, i64,
                                            vp, vp, vp, i]
        lib.oracle_atopn_calibrate.argtypes = [vp, vp, vp, i, i, i, i, i64, i, i, vp, i64, vp,
                                               vp, i]
        lib.oracle_atopn_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i64, i, i, vp, vp, i64,
                                          vp, vp, vp, vp, vp, vp, i]
        lib.oracle_sparq_attn.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i64, i, i, i, i, vp, vp,
                                          i64, vp, vp, vp, vp, vp, vp, vp, i]
        for f in (lib.oracle_topn_attn, lib.oracle_dense_attn, lib.oracle_logits,
                  lib.oracle_attend_given, lib.oracle_atopn_calibrate, lib.oracle_atopn_attn,
                  lib.oracle_sparq_attn):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _prep(q, k, v, seq_lens):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = None if v is None else np.ascontiguousarray(v)
    if q.dtype == np.float32:
        dt = 0
    elif q.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("inputs must be float32 or uint16 (bf16 bits)")
    for a in (k, v):
        if a is not None and a.dtype != q.dtype:
            raise TypeError("q, k, v must share one dtype")
    B, h_q, d = q.shape
    _, h_k, S_max, dk = k.shape
    assert dk == d and k.shape[0] == B
    h_v = h_k
    if v is not None:
        assert v.shape[0] == B and v.shape[2] == S_max and v.shape[3] == d
        h_v = v.shape[1]
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    assert lens.shape == (B,)
    return q, k, v, lens, dt, B, h_q, h_k, h_v, d, S_max


def _pairs(pairs, B, h_q):
    if pairs is None:
        return None, B * h_q
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    return pr, pr.shape[0]


def topn_attn(q, k, v, seq_lens, N, pairs=None, threads=0):
    """Top-N decode attention for all (b, i) pairs, or the listed ones.

    Returns dict: out [P][d] f64, idx [P][N] int32 (ascending, -1 pad),
    sel [P][N] f64 (-inf pad), tN [P], psum [P], threads (count used).
    """
    q, k, v, lens, dt, B, h_q, h_k, h_v, d, S = _prep(q, k, v, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    out = np.empty((P, d))
    idx = np.empty((P, N), dtype=np.int32)
    sel = np.empty((P, N))
    tN = np.empty(P)
    psum = np.empty(P)
    rc = _load().oracle_topn_attn(_p(q), _p(k), _p(v), _p(lens), B, h_q, h_k, h_v, d, S, dt,
                                  int(N), _p(pr), P, _p(out), _p(idx), _p(sel), _p(tN),
                                  _p(psum), int(threads))
    if rc < 0:
        raise ValueError("oracle_topn_attn: bad arguments")
    return {"out": out, "idx": idx, "sel": sel, "tN": tN, "psum": psum, "threads": rc}


def dense_attn(q, k, v, seq_lens, pairs=None, threads=0):
    """Full decode attention over all L_b positions. Returns (out [P][d], threads)."""
    q, k, v, lens, dt, B, h_q, h_k, h_v, d, S = _prep(q, k, v, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    out = np.empty((P, d))
    rc = _load().oracle_dense_attn(_p(q), _p(k), _p(v), _p(lens), B, h_q, h_k, h_v, d, S, dt,
                                   _p(pr), P, _p(out), int(threads))
    if rc < 0:
        raise ValueError("oracle_dense_attn: bad arguments")
    return out, rc


def logits(q, k, seq_lens, pairs=None, threads=0):
    """Scaled logits [P][S_max] in fp64, NaN at positions >= L_b."""
    q, k, _, lens, dt, B, h_q, h_k, _, d, S = _prep(q, k, None, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    sc = np.empty((P, S))
    rc = _load().oracle_logits(_p(q), _p(k), _p(lens), B, h_q, h_k, d, S, dt, _p(pr), P,
                               _p(sc), int(threads))
    if rc < 0:
        raise ValueError("oracle_logits: bad arguments")
    return sc


def attend_given(q, k, v, seq_lens, idx, pairs=None, threads=0):
    """Eq. 7 on given index sets idx [P][N] (-1 entries ignored). Returns (out, psum)."""
    q, k, v, lens, dt, B, h_q, h_k, h_v, d, S = _prep(q, k, v, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(P, -1)
    N = idx.shape[1]
    out = np.empty((P, d))
    psum = np.empty(P)
    rc = _load().oracle_attend_given(_p(q), _p(k), _p(v), _p(lens), B, h_q, h_k, h_v, d, S, dt,
                                     N, _p(pr), P, _p(idx), _p(out), _p(psum), int(threads))
    if rc < 0:
        raise ValueError("oracle_attend_given: bad arguments or invalid index set")
    return out, psum


def atopn_calibrate(q, k, seq_lens, N, pairs=None, threads=0):
    """Atop-N calibration: tau [P] (the N_eff-th largest softmax probability of
    each row, NaN if L = 0) and lse [P] (log-sum-exp of the row's logits)."""
    q, k, _, lens, dt, B, h_q, h_k, _, d, S = _prep(q, k, None, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    tau = np.empty(P)
    lse = np.empty(P)
    rc = _load().oracle_atopn_calibrate(_p(q), _p(k), _p(lens), B, h_q, h_k, d, S, dt, int(N),
                                        _p(pr), P, _p(tau), _p(lse), int(threads))
    if rc < 0:
        raise ValueError("oracle_atopn_calibrate: bad arguments")
    return tau, lse


def atopn_attn(q, k, v, seq_lens, N, tau, pairs=None, threads=0):
    """Atop-N step with stale thresholds tau [P] (one per listed pair).

    Returns dict: out [P][d], idx [P][2N] int32 (ascending, -1 pad),
    sel [P][2N] (-inf pad), above [P] (positions reaching the threshold,
    before the 2N cap), theta [P] (logit threshold), psum [P], threads.
    """
    q, k, v, lens, dt, B, h_q, h_k, h_v, d, S = _prep(q, k, v, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    tau = np.ascontiguousarray(np.asarray(tau, dtype=np.float64).reshape(-1))
    assert tau.shape == (P,)
    cap = 2 * int(N)
    out = np.empty((P, d))
    idx = np.empty((P, cap), dtype=np.int32)
    sel = np.empty((P, cap))
    above = np.empty(P, dtype=np.int64)
    theta = np.empty(P)
    psum = np.empty(P)
    rc = _load().oracle_atopn_attn(_p(q), _p(k), _p(v), _p(lens), B, h_q, h_k, h_v, d, S, dt,
                                   int(N), _p(tau), _p(pr), P, _p(out), _p(idx), _p(sel),
                                   _p(above), _p(theta), _p(psum), int(threads))
    if rc < 0:
        raise ValueError("oracle_atopn_attn: bad arguments")
    return {"out": out, "idx": idx, "sel": sel, "above": above, "theta": theta, "psum": psum,
            "threads": rc}


def sparq_attn(q, k, v, seq_lens, N, r, local=0, vmean=None, pairs=None, scores=False,
               threads=0):
    """SparQ-style step: approximate scores over the r kept query dims of the
    key head's group, the last `local` positions always kept plus the N - local
    best-scored of the rest, exact attention over the kept set, and the mean
    value reallocation when vmean [B][h_v][d] is given.

    Returns dict: out [P][d], idx [P][N] int32 (ascending, -1 pad), alpha [P],
    tau [P] (0 when the approximate scores are all 0), zthr [P] (smallest
    kept approximate score of the non-local part, NaN if none), dims [P][r]
    (ascending), zhat [P][S_max] (only with scores=True; NaN past L), threads.
    """
    q, k, v, lens, dt, B, h_q, h_k, h_v, d, S = _prep(q, k, v, seq_lens)
    pr, P = _pairs(pairs, B, h_q)
    vm = None
    if vmean is not None:
        vm = np.ascontiguousarray(np.asarray(vmean, dtype=np.float64).reshape(B, h_v, d))
    out = np.empty((P, d))
    idx = np.empty((P, N), dtype=np.int32)
    alpha = np.empty(P)
    tau = np.empty(P)
    zthr = np.empty(P)
    dims = np.empty((P, r), dtype=np.int32)
    zhat = np.empty((P, S)) if scores else None
    rc = _load().oracle_sparq_attn(_p(q), _p(k), _p(v), _p(lens), B, h_q, h_k, h_v, d, S, dt,
                                   int(N), int(r), int(local), _p(vm), _p(pr), P, _p(out),
                                   _p(idx), _p(alpha), _p(tau), _p(zthr), _p(dims), _p(zhat),
                                   int(threads))
    if rc < 0:
        raise ValueError("oracle_sparq_attn: bad arguments")
    res = {"out": out, "idx": idx, "alpha": alpha, "tau": tau, "zthr": zthr, "dims": dims,
           "threads": rc}
    if scores:
        res["zhat"] = zhat
    return res
