"""Tensor-level wrappers over the libsaga C ABI.

PyTorch supplies device memory and the current HIP stream; shapes and the
dtype are read from the tensors and passed to the C entry points unchanged.
These wrappers allocate the output and the workspace when the caller does
not pass them (outside libsaga, which itself never allocates).
"""
from __future__ import annotations

import torch

from . import _binding as C


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return C.SAGA_F32
    if t.dtype == torch.bfloat16:
        return C.SAGA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _shapes(q, k_cache, v_cache, seq_lens):
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    B, h_q, d = q.shape
    kb, h_k, S_max, kd = k_cache.shape
    if kb != B or kd != d:
        raise ValueError("k_cache must be [B][h_k][S_max][d]")
    h_v = h_k
    if v_cache is not None:
        vb, h_v, vS, vd = v_cache.shape
        if vb != B or vS != S_max or vd != d:
            raise ValueError("v_cache must be [B][h_v][S_max][d]")
        if v_cache.dtype != q.dtype:
            raise TypeError("q, k_cache and v_cache must share one dtype")
    if k_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be [B]")
    return B, h_q, h_k, h_v, d, S_max


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def workspace_size(q, k_cache, v_cache, seq_lens, N) -> int:
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    return C.saga_workspace_size(B, h_q, h_k, h_v, d, N, S, _dtype_code(q))


def dense_workspace_size(q, k_cache, v_cache, seq_lens) -> int:
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    return C.saga_dense_workspace_size(B, h_q, h_k, h_v, d, S, _dtype_code(q))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator hands out blocks aligned well beyond 256 bytes
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def decode_attn(q, k_cache, v_cache, seq_lens, N, *, out=None, workspace=None, idx_out=None,
                stream=None):
    """SAGA top-N decode attention; returns out (float32 [B][h_q][d])."""
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    dt = _dtype_code(q)
    need = C.saga_workspace_size(B, h_q, h_k, h_v, d, N, S, dt)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    st = C.saga_decode_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                            _stream(stream), S, dt, workspace, workspace.numel(), idx_out)
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_decode_attn")
    return out


def dense_attn(q, k_cache, v_cache, seq_lens, *, out=None, workspace=None, stream=None):
    """Full decode attention (GQA when h_k == h_v, SAGA-full when h_k < h_v)."""
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    dt = _dtype_code(q)
    need = C.saga_dense_workspace_size(B, h_q, h_k, h_v, d, S, dt)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    st = C.saga_dense_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d,
                           _stream(stream), S, dt, workspace, workspace.numel())
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_dense_attn")
    return out


def debug_scores(q, k_cache, seq_lens, *, out=None, stream=None):
    """fp32 logits [B][h_q][S_max] from the K-scan kernel alone (t >= L_b untouched)."""
    B, h_q, h_k, _, d, S = _shapes(q, k_cache, None, seq_lens)
    if out is None:
        out = torch.full((B, h_q, S), float("nan"), dtype=torch.float32, device=q.device)
    st = C.saga_debug_scores(q, k_cache, seq_lens, out, B, h_q, h_k, d, _stream(stream), S,
                             _dtype_code(q))
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_debug_scores")
    return out


def atopn_workspace_size(q, k_cache, v_cache, seq_lens, N) -> int:
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    return C.saga_atopn_workspace_size(B, h_q, h_k, h_v, d, N, S, _dtype_code(q))


def atopn_calibrate(q, k_cache, v_cache, seq_lens, N, *, tau=None, out=None, workspace=None,
                    idx_out=None, stream=None):
    """Atop-N calibration step: the exact top-N step; returns (out, tau [B][h_q] float32)."""
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    dt = _dtype_code(q)
    if workspace is None:
        workspace = new_workspace(C.saga_atopn_workspace_size(B, h_q, h_k, h_v, d, N, S, dt),
                                  q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    if tau is None:
        tau = torch.empty((B, h_q), dtype=torch.float32, device=q.device)
    st = C.saga_atopn_calibrate(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                                _stream(stream), S, dt, workspace, workspace.numel(), tau,
                                idx_out)
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_atopn_calibrate")
    return out, tau


def atopn_attn(q, k_cache, v_cache, seq_lens, N, tau, *, out=None, workspace=None, idx_out=None,
               count_out=None, stream=None):
    """Atop-N step with the stale thresholds tau [B][h_q]; returns out."""
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    dt = _dtype_code(q)
    if workspace is None:
        workspace = new_workspace(C.saga_atopn_workspace_size(B, h_q, h_k, h_v, d, N, S, dt),
                                  q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    st = C.saga_atopn_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                           _stream(stream), S, dt, workspace, workspace.numel(), tau, idx_out,
                           count_out)
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_atopn_attn")
    return out


def sparq_workspace_size(q, k_cache, v_cache, seq_lens, N, r) -> int:
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    return C.saga_sparq_workspace_size(B, h_q, h_k, h_v, d, N, r, S, _dtype_code(q))


def sparq_attn(q, k_cache, kt_cache, v_cache, seq_lens, N, r, local=0, *, v_mean=None, out=None,
               workspace=None, idx_out=None, alpha_out=None, dims_out=None, stream=None):
    """SparQ-style step: approximate scores over r query dims from kt_cache
    ([B][h_k][d][S_max], the keys S-contiguous), the last `local` positions
    always kept, exact attention over the kept set, optional mean-value mix
    with v_mean (float32 [B][h_v][d]). Returns out (float32 [B][h_q][d])."""
    B, h_q, h_k, h_v, d, S = _shapes(q, k_cache, v_cache, seq_lens)
    if tuple(kt_cache.shape) != (B, h_k, d, S) or kt_cache.dtype != q.dtype:
        raise ValueError("kt_cache must be [B][h_k][d][S_max] in the cache dtype")
    if not kt_cache.is_cuda or not kt_cache.is_contiguous():
        raise ValueError("kt_cache must be a contiguous device tensor")
    if v_mean is not None and (v_mean.dtype != torch.float32 or tuple(v_mean.shape) != (B, h_v, d)
                               or not v_mean.is_cuda or not v_mean.is_contiguous()):
        raise ValueError("v_mean must be a contiguous float32 device tensor [B][h_v][d]")
    dt = _dtype_code(q)
    if workspace is None:
        workspace = new_workspace(C.saga_sparq_workspace_size(B, h_q, h_k, h_v, d, N, r, S, dt),
                                  q.device)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    st = C.saga_sparq_attn(q, k_cache, kt_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N,
                           r, local, v_mean, _stream(stream), S, dt, workspace, workspace.numel(),
                           idx_out, alpha_out, dims_out)
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_sparq_attn")
    return out


_STRATEGIES = {"logit": C.SAGA_MERGE_LOGIT, "key": C.SAGA_MERGE_KEY,
               "sequential": C.SAGA_MERGE_SEQUENTIAL}


def key_merge_workspace_size(L, D, h_q, h_kt, d) -> int:
    return C.saga_key_merge_workspace_size(L, D, h_q, h_kt, d)


def key_merge(x, wq, wk, h_q, h_kt, strategy="logit", *, workspace=None, pair_w=None,
              objective=None, stats=None, stream=None):
    """GQA -> SAGA key-head merge of one attention module (bf16 device tensors
    x [L][D], wq [h_q*d][D], wk [h_kt*d][D]). Returns (merged_k float32
    [h_kt/2][d][D], sigma int32 [h_kt]); pair_w (float64 [h_kt][h_kt]),
    objective (float64 [1]) and stats (float32 [h_kt*d*d + (h_kt*d)^2]) are
    filled when given."""
    for name, t in (("x", x), ("wq", wq), ("wk", wk)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    L, D = x.shape
    if wq.shape[1] != D or wk.shape[1] != D or wq.shape[0] % h_q or wk.shape[0] % h_kt:
        raise ValueError("wq must be [h_q*d][D] and wk [h_kt*d][D]")
    d = wq.shape[0] // h_q
    if wk.shape[0] != h_kt * d:
        raise ValueError("wq and wk head dimensions differ")
    if workspace is None:
        n = C.saga_key_merge_workspace_size(L, D, h_q, h_kt, d)
        if n == 0:
            raise C.SagaError(C.SAGA_ERR_UNSUPPORTED, "saga_key_merge_workspace_size")
        workspace = new_workspace(n, x.device)
    merged = torch.empty((h_kt // 2, d, D), dtype=torch.float32, device=x.device)
    sigma = torch.empty((h_kt,), dtype=torch.int32, device=x.device)
    st = C.saga_key_merge(x, wq, wk, L, D, h_q, h_kt, d, _STRATEGIES[strategy], C.SAGA_BF16,
                          merged, sigma, pair_w, objective, stats, workspace, workspace.numel(),
                          _stream(stream))
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_key_merge")
    return merged, sigma


def merge_permute(sigma, wq, wv, wo, h_q, h_kt, *, stream=None):
    """App. B's induced permutations: returns (wq', wv', wo') for the pairing
    sigma (int32 device [h_kt]); wq [h_q*d][D], wv [h_kt*d][D], wo [D][h_q*d]."""
    D = wq.shape[1]
    d = wq.shape[0] // h_q
    dt = _dtype_code(wq)
    for t in (wq, wv, wo):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != wq.dtype:
            raise ValueError("weights must be contiguous device tensors of one dtype")
    outs = [torch.empty_like(t) for t in (wq, wv, wo)]
    st = C.saga_merge_permute(sigma, wq, wv, wo, D, h_q, h_kt, d, dt, *outs, _stream(stream))
    if st != C.SAGA_OK:
        raise C.SagaError(st, "saga_merge_permute")
    return tuple(outs)
