"""ctypes binding of libsaga (argument marshalling only).

The functions named like the C entry points take the same arguments, with
device pointers given as ints (or torch tensors, whose data_ptr() is used)
and the stream as an int handle. Every step of the computation runs in the
HIP kernels of libsaga.so; there is no fallback: if the library is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsaga.so")

SAGA_OK = 0
SAGA_ERR_INVALID_ARG = -1
SAGA_ERR_UNSUPPORTED = -2
SAGA_ERR_WORKSPACE = -3
SAGA_ERR_HIP = -4
SAGA_ERR_TOO_LARGE = -5
SAGA_F32 = 0
SAGA_BF16 = 1

EXPORTS = ("saga_workspace_size", "saga_decode_attn", "saga_decode_attn_timed",
           "saga_noalloc_scratch_bytes", "saga_decode_attn_noalloc",
           "saga_dense_workspace_size", "saga_atopn_workspace_size", "saga_atopn_calibrate",
           "saga_atopn_attn", "saga_sparq_workspace_size", "saga_sparq_attn",
           "saga_dense_attn", "saga_debug_scores", "saga_debug_fallback_rows",
           "saga_debug_stream_read", "saga_debug_gather_rows",
           "saga_key_merge_workspace_size", "saga_key_merge", "saga_key_merge_timed",
           "saga_merge_permute", "saga_status_string")


class SagaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime (libamdhip64.so, same SONAME as ROCm's).
    # Streams and device pointers handed to libsaga come from torch, so torch
    # must be loaded first: libsaga's libamdhip64.so.7 dependency then binds to
    # that same runtime instead of loading a second copy that sees no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run sparse_asymmetric_gqa_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.saga_workspace_size.argtypes = [i, i, i, i, i, i, i64, i]
    lib.saga_workspace_size.restype = sz
    lib.saga_dense_workspace_size.argtypes = [i, i, i, i, i, i64, i]
    lib.saga_dense_workspace_size.restype = sz
    lib.saga_decode_attn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i64, i, vp, sz, vp]
    lib.saga_decode_attn.restype = i
    lib.saga_decode_attn_timed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i64, i, vp,
                                           sz, vp, vp, i]
    lib.saga_decode_attn_timed.restype = i
    lib.saga_noalloc_scratch_bytes.argtypes = []
    lib.saga_noalloc_scratch_bytes.restype = sz
    lib.saga_decode_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i64, i, vp]
    lib.saga_decode_attn_noalloc.restype = i
    lib.saga_dense_attn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i64, i, vp, sz]
    lib.saga_dense_attn.restype = i
    lib.saga_debug_scores.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, i64, i]
    lib.saga_debug_scores.restype = i
    lib.saga_debug_fallback_rows.argtypes = [vp, sz, i, i, i, i, i, i, i64, i, vp, vp]
    lib.saga_debug_fallback_rows.restype = i
    lib.saga_debug_stream_read.argtypes = [vp, sz, vp, vp]
    lib.saga_debug_stream_read.restype = i
    lib.saga_debug_gather_rows.argtypes = [vp, vp, vp, i, i, i, i, i, vp, i64, i]
    lib.saga_debug_gather_rows.restype = i
    lib.saga_atopn_workspace_size.argtypes = [i, i, i, i, i, i, i64, i]
    lib.saga_atopn_workspace_size.restype = sz
    lib.saga_atopn_calibrate.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i64, i, vp, sz,
                                         vp, vp]
    lib.saga_atopn_calibrate.restype = i
    lib.saga_atopn_attn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i64, i, vp, sz, vp,
                                    vp, vp]
    lib.saga_atopn_attn.restype = i
    lib.saga_sparq_workspace_size.argtypes = [i, i, i, i, i, i, i, i64, i]
    lib.saga_sparq_workspace_size.restype = sz
    lib.saga_sparq_attn.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i64,
                                    i, vp, sz, vp, vp, vp]
    lib.saga_sparq_attn.restype = i
    lib.saga_key_merge_workspace_size.argtypes = [i64, i, i, i, i]
    lib.saga_key_merge_workspace_size.restype = sz
    lib.saga_key_merge.argtypes = [vp, vp, vp, i64, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, sz,
                                   vp]
    lib.saga_key_merge.restype = i
    lib.saga_key_merge_timed.argtypes = [vp, vp, vp, i64, i, i, i, i, i, i, vp, vp, vp, vp, vp,
                                         vp, sz, vp, vp, i]
    lib.saga_key_merge_timed.restype = i
    lib.saga_merge_permute.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp]
    lib.saga_merge_permute.restype = i
    lib.saga_status_string.argtypes = [i]
    lib.saga_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def status_string(status: int) -> str:
    return lib.saga_status_string(int(status)).decode()


def saga_status_string(status: int) -> str:
    return status_string(status)


def saga_workspace_size(B, h_q, h_k, h_v, d, N, S_max, dtype) -> int:
    return int(lib.saga_workspace_size(B, h_q, h_k, h_v, d, N, S_max, dtype))


def saga_dense_workspace_size(B, h_q, h_k, h_v, d, S_max, dtype) -> int:
    return int(lib.saga_dense_workspace_size(B, h_q, h_k, h_v, d, S_max, dtype))


def saga_decode_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream,
                     S_max, dtype, workspace, workspace_bytes, idx_out=None) -> int:
    return int(lib.saga_decode_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                    _ptr(out), B, h_q, h_k, h_v, d, N, _ptr(stream), S_max,
                                    dtype, _ptr(workspace), workspace_bytes, _ptr(idx_out)))


def saga_decode_attn_timed(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream,
                           S_max, dtype, workspace, workspace_bytes, idx_out, events) -> int:
    """events: a sequence of 0..4 raw hipEvent_t handles (ints)."""
    n = len(events)
    arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(e)) for e in events])
    return int(lib.saga_decode_attn_timed(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                          _ptr(out), B, h_q, h_k, h_v, d, N, _ptr(stream), S_max,
                                          dtype, _ptr(workspace), workspace_bytes,
                                          _ptr(idx_out), arr, n))


def saga_noalloc_scratch_bytes() -> int:
    return int(lib.saga_noalloc_scratch_bytes())


def saga_decode_attn_noalloc(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream,
                             S_max, dtype, idx_out=None) -> int:
    return int(lib.saga_decode_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(seq_lens), _ptr(out), B, h_q, h_k, h_v, d, N,
                                            _ptr(stream), S_max, dtype, _ptr(idx_out)))


def saga_dense_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, stream, S_max,
                    dtype, workspace, workspace_bytes) -> int:
    return int(lib.saga_dense_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                   _ptr(out), B, h_q, h_k, h_v, d, _ptr(stream), S_max, dtype,
                                   _ptr(workspace), workspace_bytes))


def saga_debug_scores(q, k_cache, seq_lens, scores, B, h_q, h_k, d, stream, S_max,
                      dtype) -> int:
    return int(lib.saga_debug_scores(_ptr(q), _ptr(k_cache), _ptr(seq_lens), _ptr(scores), B,
                                     h_q, h_k, d, _ptr(stream), S_max, dtype))


def saga_debug_fallback_rows(workspace, workspace_bytes, B, h_q, h_k, h_v, d, N, S_max, dtype,
                             host_flags, stream) -> int:
    """host_flags: a writable int32 numpy array of B*h_q entries (host memory)."""
    return int(lib.saga_debug_fallback_rows(_ptr(workspace), workspace_bytes, B, h_q, h_k, h_v,
                                            d, N, S_max, dtype,
                                            ctypes.c_void_p(host_flags.ctypes.data), _ptr(stream)))


def saga_debug_stream_read(buf, nbytes, sink, stream) -> int:
    return int(lib.saga_debug_stream_read(_ptr(buf), nbytes, _ptr(sink), _ptr(stream)))


def saga_debug_gather_rows(v_cache, idx, out, B, h_q, h_v, d, N, stream, S_max, dtype) -> int:
    return int(lib.saga_debug_gather_rows(_ptr(v_cache), _ptr(idx), _ptr(out), B, h_q, h_v, d,
                                          N, _ptr(stream), S_max, dtype))


def saga_atopn_workspace_size(B, h_q, h_k, h_v, d, N, S_max, dtype) -> int:
    return int(lib.saga_atopn_workspace_size(B, h_q, h_k, h_v, d, N, S_max, dtype))


def saga_atopn_calibrate(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream,
                         S_max, dtype, workspace, workspace_bytes, tau, idx_out=None) -> int:
    return int(lib.saga_atopn_calibrate(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                        _ptr(out), B, h_q, h_k, h_v, d, N, _ptr(stream), S_max,
                                        dtype, _ptr(workspace), workspace_bytes, _ptr(tau),
                                        _ptr(idx_out)))


def saga_atopn_attn(q, k_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, stream, S_max,
                    dtype, workspace, workspace_bytes, tau, idx_out=None, count_out=None) -> int:
    return int(lib.saga_atopn_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                   _ptr(out), B, h_q, h_k, h_v, d, N, _ptr(stream), S_max, dtype,
                                   _ptr(workspace), workspace_bytes, _ptr(tau), _ptr(idx_out),
                                   _ptr(count_out)))


def saga_sparq_workspace_size(B, h_q, h_k, h_v, d, N, r, S_max, dtype) -> int:
    return int(lib.saga_sparq_workspace_size(B, h_q, h_k, h_v, d, N, r, S_max, dtype))


def saga_sparq_attn(q, k_cache, kt_cache, v_cache, seq_lens, out, B, h_q, h_k, h_v, d, N, r,
                    local, v_mean, stream, S_max, dtype, workspace, workspace_bytes, idx_out=None,
                    alpha_out=None, dims_out=None) -> int:
    return int(lib.saga_sparq_attn(_ptr(q), _ptr(k_cache), _ptr(kt_cache), _ptr(v_cache),
                                   _ptr(seq_lens), _ptr(out), B, h_q, h_k, h_v, d, N, r, local,
                                   _ptr(v_mean), _ptr(stream), S_max, dtype, _ptr(workspace),
                                   workspace_bytes, _ptr(idx_out), _ptr(alpha_out),
                                   _ptr(dims_out)))


SAGA_MERGE_LOGIT, SAGA_MERGE_KEY, SAGA_MERGE_SEQUENTIAL = 0, 1, 2


def saga_key_merge_workspace_size(L, D, h_q, h_kt, d) -> int:
    return int(lib.saga_key_merge_workspace_size(L, D, h_q, h_kt, d))


def saga_key_merge(x, wq, wk, L, D, h_q, h_kt, d, strategy, dtype, merged_k, sigma, pair_w,
                   objective, stats, workspace, workspace_bytes, stream) -> int:
    return int(lib.saga_key_merge(_ptr(x), _ptr(wq), _ptr(wk), L, D, h_q, h_kt, d, strategy,
                                  dtype, _ptr(merged_k), _ptr(sigma), _ptr(pair_w),
                                  _ptr(objective), _ptr(stats), _ptr(workspace),
                                  workspace_bytes, _ptr(stream)))


def saga_key_merge_timed(x, wq, wk, L, D, h_q, h_kt, d, strategy, dtype, merged_k, sigma,
                         pair_w, objective, stats, workspace, workspace_bytes, stream, events,
                         n_events=None) -> int:
    """events: a sequence of hipEvent_t handles (ints), or None."""
    if events is None:
        arr, n = None, int(n_events or 0)
    else:
        n = len(events) if n_events is None else int(n_events)
        arr = (ctypes.c_void_p * max(1, len(events)))(*[ctypes.c_void_p(int(e)) for e in events])
    return int(lib.saga_key_merge_timed(_ptr(x), _ptr(wq), _ptr(wk), L, D, h_q, h_kt, d,
                                        strategy, dtype, _ptr(merged_k), _ptr(sigma),
                                        _ptr(pair_w), _ptr(objective), _ptr(stats),
                                        _ptr(workspace), workspace_bytes, _ptr(stream),
                                        arr, n))


def saga_merge_permute(sigma, wq, wv, wo, D, h_q, h_kt, d, dtype, wq_out, wv_out, wo_out,
                       stream) -> int:
    return int(lib.saga_merge_permute(_ptr(sigma), _ptr(wq), _ptr(wv), _ptr(wo), D, h_q, h_kt,
                                      d, dtype, _ptr(wq_out), _ptr(wv_out), _ptr(wo_out),
                                      _ptr(stream)))
