"""saga_decode_attn_noalloc (the entry point that allocates nothing, its
scratch a static device array of the library) against saga_decode_attn with
a caller workspace, through the C ABI: two calls in a row on one GPU, the
second with a smaller input, each must give the same kept index sets and
the same outputs (the same kernels run on the same inputs, so bitwise)."""
import numpy as np
import pytest
import torch

import synth
from parity_helpers import to_device

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_asymmetric_gqa_amd as saga  # noqa: E402


def _both(case, N):
    print(f"[noalloc] B={case.B} h_q={case.h_q} h_k={case.h_k} h_v={case.h_v} d={case.d} "
          f"S={case.S_max} N={N} {case.dtype}", flush=True)
    x = synth.make_inputs(case)
    dx = to_device(x)
    B, h_q, h_k, h_v, d, S = case.B, case.h_q, case.h_k, case.h_v, case.d, case.S_max
    dt = saga.SAGA_F32 if case.dtype == "f32" else saga.SAGA_BF16
    st = torch.cuda.current_stream().cuda_stream
    wsb = saga.saga_workspace_size(B, h_q, h_k, h_v, d, N, S, dt)
    assert 0 < wsb <= saga.saga_noalloc_scratch_bytes()
    ws = saga.new_workspace(wsb, "cuda")
    ref_out = torch.empty((B, h_q, d), dtype=torch.float32, device="cuda")
    ref_idx = torch.empty((B, h_q, N), dtype=torch.int32, device="cuda")
    assert saga.saga_decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], ref_out, B, h_q, h_k,
                                 h_v, d, N, st, S, dt, ws, wsb, ref_idx) == saga.SAGA_OK
    out = torch.full((B, h_q, d), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, h_q, N), -7, dtype=torch.int32, device="cuda")
    assert saga.saga_decode_attn_noalloc(dx["q"], dx["k"], dx["v"], dx["seq_lens"], out, B, h_q,
                                         h_k, h_v, d, N, st, S, dt, idx) == saga.SAGA_OK
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ref_idx.cpu())
    assert torch.equal(out.cpu(), ref_out.cpu())
    assert np.isfinite(out.cpu().numpy()).all()


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    big = synth.CASES["llama32_1b_8to4"]
    _both(big, big.N)
    small = synth.small_case(B=3, h_q=12, h_k=1, h_v=2, d=128, S_max=2049, N=300,
                             dtype="bf16", ragged=True, seed=91)
    _both(small, 300)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    q = torch.zeros((64, 12, 128), dtype=torch.bfloat16, device="cuda")
    lens = torch.ones((64,), dtype=torch.int32, device="cuda")
    out = torch.empty((64, 12, 128), dtype=torch.float32, device="cuda")
    S = 1 << 20   # the caches are never read: the call is refused on the host
    rc = saga.saga_decode_attn_noalloc(q, q, q, lens, out, 64, 12, 1, 2, 128, 1024,
                                       torch.cuda.current_stream().cuda_stream, S,
                                       saga.SAGA_BF16, None)
    assert rc == saga.SAGA_ERR_TOO_LARGE
