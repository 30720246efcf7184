"""GPU parity: libsaga (HIP, gfx950) against the fp64 CPU oracle.

Every call goes through the C ABI (sparse_asymmetric_gqa_amd._binding via the
tensor wrappers). Index sets must match the oracle exactly apart from
near-threshold ties (see parity_helpers); outputs must be within 2e-3 (bf16
inputs) or 1e-5 (fp32 inputs) of the oracle on the GPU's own kept set.
The five workloads run at their full sizes and every (b, i) row of every
workload is compared, the largest in the launch configuration the benchmark
times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_helpers import all_pairs, check_index_sets, check_outputs, to_device, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import sparse_asymmetric_gqa_amd as saga  # noqa: E402  (fails loudly if not built)


def _say(*a):
    print(*a, flush=True)


def _run_decode(x, dx, case, N, pairs, label):
    _say(f"[decode] {label}: B={case.B} h_q={case.h_q} h_k={case.h_k} h_v={case.h_v} "
         f"d={case.d} S={case.S_max} N={N} {case.dtype}")
    idx = torch.empty((case.B, case.h_q, N), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N, idx_out=idx)
    torch.cuda.synchronize()
    rows = [b * case.h_q + i for b, i in pairs]
    g_idx = idx.reshape(-1, N).cpu().numpy()[rows]
    g_out = out.reshape(-1, case.d).cpu().numpy()[rows]
    ref = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], N, pairs=pairs)
    nbad, ndiff = check_index_sets(g_idx, ref, x, pairs, N)
    err = check_outputs(g_out, g_idx, x, pairs, tol_for(case.dtype))
    if nbad == 0:
        err2 = np.abs(g_out - ref["out"]).max()
        assert err2 <= tol_for(case.dtype), err2
    _say(f"    rows={len(pairs)} differing-rows={nbad} sym-diff={ndiff} max|err|={err:.2e}")
    return g_idx, g_out


WORKLOADS = ["tiny_fp32", "llama32_1b_8to4", "qwen25_1p5b_2to1_ragged", "smollm2_360m_1x8",
             "qwen25_1p5b_b64_32k"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_decode_workloads(name):
    case = synth.CASES[name]
    x = synth.make_inputs(case)
    dx = to_device(x)
    Ns = synth.SMOLLM_N_SWEEP if name == "smollm2_360m_1x8" else (case.N,)
    pairs = all_pairs(case.B, case.h_q)
    for N in Ns:
        _run_decode(x, dx, case, N, pairs, name)


@pytest.mark.parametrize("name", list(synth.DENSE_BASELINES))
def test_dense_baselines(name):
    base = synth.CASES[name]
    for (hk, hv) in synth.DENSE_BASELINES[name]:
        case = base.with_heads(hk, hv, seed=100 + base.seed)
        _say(f"[dense] {name} ({hk},{hv})")
        x = synth.make_inputs(case)
        dx = to_device(x)
        out = saga.dense_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"])
        torch.cuda.synchronize()
        pairs = all_pairs(case.B, case.h_q)
        rows = [b * case.h_q + i for b, i in pairs]
        ref, _ = oracle.dense_attn(x["q"], x["k"], x["v"], x["seq_lens"], pairs=pairs)
        err = np.abs(out.reshape(-1, case.d).cpu().numpy()[rows] - ref).max()
        _say(f"    rows={len(pairs)} max|err|={err:.2e}")
        assert err <= tol_for(case.dtype)
        del dx
        torch.cuda.empty_cache()


DENSE_SMALL = [
    # (B, h_q, h_k, h_v, d, S_max, dtype, lens)
    (3, 6, 2, 3, 64, 700, "bf16", [700, 513, 1]),       # a value head spans two key heads
    (2, 12, 1, 2, 128, 1300, "bf16", [1300, 511]),      # SAGA (1, 2), partial chunks
    (2, 8, 4, 4, 128, 300, "f32", [300, 17]),           # GQA, fp32, rows shorter than a chunk
    (1, 32, 1, 4, 64, 900, "bf16", [900]),              # key group of 32 (256-position chunks)
    (1, 64, 1, 2, 128, 600, "f32", [600]),              # key group of 64, value group of 32
    (2, 16, 1, 8, 64, 1024, "bf16", [1024, 0]),         # empty row -> 0
    # shapes whose item count picks the longer chunks (1024 and 512 positions)
    (8, 8, 4, 4, 128, 8500, "bf16", [8500, 5000, 1025, 1024, 1023, 1, 0, 3000]),
    (2, 4, 2, 2, 128, 33000, "bf16", [33000, 16385]),   # 512 positions, 65 partials per row
    (16, 4, 1, 2, 64, 17000, "f32",
     [17000, 16999, 9000, 1024, 1025, 2048, 1, 511, 513, 4000, 17000, 300, 12000, 7, 15000, 0]),
]


@pytest.mark.parametrize("shape", DENSE_SMALL)
def test_dense_small_shapes(shape):
    B, h_q, h_k, h_v, d, S, dt, lens = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=1, dtype=dt, seed=67)
    lens = np.array(lens, np.int32)
    x = synth.make_inputs(case, np.maximum(lens, 1))
    x["seq_lens"] = lens
    _say(f"[dense] small {shape}")
    dx = to_device(x)
    out = saga.dense_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"]).reshape(-1, d).cpu().numpy()
    live = [(b, i) for b in range(B) for i in range(h_q) if lens[b] > 0]
    ref, _ = oracle.dense_attn(x["q"], x["k"], x["v"], np.maximum(lens, 1), pairs=live)
    err = np.abs(out[[b * h_q + i for b, i in live]] - ref).max()
    _say(f"    max|err|={err:.2e}")
    assert err <= tol_for(dt)
    for b in range(B):
        if lens[b] == 0:
            assert not out[b * h_q:(b + 1) * h_q].any()


SMALL = [
    # (B, h_q, h_k, h_v, d, S_max, N, dtype, ragged)
    (2, 8, 2, 4, 64, 1030, 100, "bf16", True),
    (2, 8, 2, 4, 128, 1030, 100, "f32", True),
    (1, 4, 1, 2, 64, 777, 64, "f32", False),
    (3, 12, 1, 2, 128, 2049, 300, "bf16", True),
    (2, 6, 2, 2, 64, 513, 37, "bf16", False),       # h_k == h_v (GQA)
    (1, 64, 1, 2, 64, 600, 50, "bf16", False),      # key group of 64, value group of 32
    (2, 32, 2, 32, 128, 300, 16, "bf16", False),    # g_v = 1
    (1, 16, 1, 8, 64, 4100, 1000, "bf16", False),   # select tile KPT=8
]


@pytest.mark.parametrize("shape", SMALL)
def test_decode_small_shapes(shape):
    B, h_q, h_k, h_v, d, S, N, dt, ragged = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype=dt,
                            ragged=ragged, seed=41)
    x = synth.make_inputs(case)
    _run_decode(x, to_device(x), case, N, all_pairs(B, h_q), f"small{shape}")


SMALL_BATCH = [
    # (B, h_q, h_k, h_v, d, S_max, N, ragged): few K-scan items of 1024 positions
    # (256-position items) and few rows (the value gather split along each
    # row's kept list, merged by the part that finishes last)
    (1, 12, 1, 2, 128, 8192, 1024, False),
    (1, 12, 1, 2, 128, 65536, 1024, False),
    (4, 12, 2, 2, 128, 16384, 1024, False),
    (2, 12, 1, 2, 128, 40000, 2048, True),
    (1, 4, 1, 2, 64, 300, 64, False),
    (3, 16, 1, 8, 64, 5000, 512, True),
    # rows that give every split count from 2 to 7 (256 / rows parts per row)
    (8, 12, 1, 2, 128, 3000, 512, True),     # 96 rows: 2 parts
    (5, 16, 1, 2, 64, 2000, 256, True),      # 80 rows: 3 parts
    (4, 16, 2, 4, 64, 2500, 300, True),      # 64 rows: 4 parts
    (4, 12, 1, 2, 128, 3000, 512, True),     # 48 rows: 5 parts
    (5, 8, 1, 2, 128, 1500, 200, False),     # 40 rows: 6 parts
    (3, 12, 1, 2, 64, 4000, 700, False),     # 36 rows: 7 parts
    # 512-position K-scan items: 1024-position ones would leave CUs idle, and
    # rows longer than 64 Ki positions do not fit 256 items of 256
    (4, 12, 1, 2, 128, 32768, 1024, True),
    (1, 12, 1, 2, 128, 100000, 1024, True),
]


@pytest.mark.parametrize("shape", SMALL_BATCH)
def test_small_batch_shapes(shape):
    B, h_q, h_k, h_v, d, S, N, ragged = shape
    case = synth.small_case(B=B, h_q=h_q, h_k=h_k, h_v=h_v, d=d, S_max=S, N=N, dtype="bf16",
                            ragged=ragged, seed=97)
    x = synth.make_inputs(case)
    dx = to_device(x)
    g1, o1 = _run_decode(x, dx, case, N, all_pairs(B, h_q), f"small-batch{shape}")
    # the same call again gives the same bits (the merge order is fixed)
    idx = torch.empty((B, h_q, N), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N, idx_out=idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.reshape(-1, N).cpu().numpy(), g1)
    assert np.array_equal(out.reshape(-1, d).cpu().numpy(), o1)


@pytest.mark.parametrize("h_q", [4, 32])
def test_select_multi_tile_rows(h_q):
    # rows longer than one register tile of the selector take the tiled path that
    # re-reads keys each round: the dense selector (key group of 32: 32768 keys per
    # tile) and the union selector's dense fallback / multi-tile candidate sets
    case = synth.small_case(B=1, h_q=h_q, h_k=1, h_v=2, d=64, S_max=40000, N=700,
                            dtype="bf16", seed=43)
    lens = np.array([39999], np.int32)
    x = synth.make_inputs(case, lens)
    _run_decode(x, to_device(x), case, 700, all_pairs(1, h_q), "multi-tile")


def test_union_rows_routed_to_the_general_code():
    # q = 0: every logit ties, each chunk list holds all 1024 keys, longer than
    # the union selector's register runs -> general code; the first N positions
    # win the ties
    case = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=5000, N=1000, dtype="bf16",
                            seed=59)
    x = synth.make_inputs(case)
    x["q"][:] = 0
    g_idx, _ = _run_decode(x, to_device(x), case, 1000, all_pairs(1, 4), "q=0 long")
    assert all(list(g_idx[r]) == list(range(1000)) for r in range(4))
    # more than 256 chunks in a row -> general code
    case = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=263000, N=512, dtype="bf16",
                            seed=61)
    x = synth.make_inputs(case)
    _run_decode(x, to_device(x), case, 512, all_pairs(1, 4), "257 chunks")


def test_rows_beyond_the_union_path():
    # more than 512 chunks of 1024 positions: the decode call takes the dense
    # logit path (K-scan to fp32 logits, dense select, sparse PV) even for a key
    # group of 12; one row of 600000 positions, one just past the limit
    case = synth.small_case(B=2, h_q=12, h_k=1, h_v=2, d=64, S_max=600000, N=1024,
                            dtype="bf16", seed=67)
    lens = np.array([600000, 524289], np.int32)
    x = synth.make_inputs(case, lens)
    _run_decode(x, to_device(x), case, 1024, all_pairs(2, 12), "beyond union path")


def test_ragged_edge_lengths_and_nan_tail():
    case = synth.small_case(B=10, h_q=4, h_k=1, h_v=2, d=64, S_max=1030, N=16, dtype="bf16",
                            seed=47)
    lens = np.array([1, 15, 16, 17, 255, 1000, 1023, 1024, 1025, 1030], np.int32)
    x = synth.make_inputs(case, lens)
    g_idx, g_out = _run_decode(x, to_device(x), case, 16, all_pairs(10, 4), "ragged")
    # cache rows past L_b filled with NaN must not change anything
    xn = {k: v.copy() for k, v in x.items()}
    for b, L in enumerate(lens):
        xn["k"][b, :, L:] = 0x7FC0
        xn["v"][b, :, L:] = 0x7FC0
    dn = to_device(xn)
    idx = torch.empty((10, 4, 16), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dn["q"], dn["k"], dn["v"], dn["seq_lens"], 16, idx_out=idx)
    assert np.array_equal(idx.reshape(-1, 16).cpu().numpy(), g_idx)
    assert np.array_equal(out.reshape(-1, 64).cpu().numpy(), g_out)


def test_zero_query_ties_and_N_edges():
    case = synth.small_case(B=2, h_q=8, h_k=2, h_v=4, d=128, S_max=500, N=40, dtype="bf16",
                            seed=53)
    lens = np.array([500, 33], np.int32)
    x = synth.make_inputs(case, lens)
    x["q"][:] = 0
    g_idx, g_out = _run_decode(x, to_device(x), case, 40, all_pairs(2, 8), "q=0")
    for r in range(16):
        n = min(40, int(lens[r // 8]))
        assert list(g_idx[r, :n]) == list(range(n))
    x = synth.make_inputs(case, lens)
    dx = to_device(x)
    for N in (1, 2, 499, 500, 501, 4096):
        _run_decode(x, dx, case, N, all_pairs(2, 8), f"N={N}")
    # N >= L_b is full attention
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 4096)
    ref, _ = oracle.dense_attn(x["q"], x["k"], x["v"], lens)
    assert np.abs(out.reshape(-1, 128).cpu().numpy() - ref).max() <= 2e-3


def test_duplicated_key_row_at_threshold_goes_to_lower_position():
    case = synth.small_case(B=1, h_q=1, h_k=1, h_v=1, d=64, S_max=300, N=20, dtype="bf16",
                            seed=59)
    x = synth.make_inputs(case)
    sc = oracle.logits(x["q"], x["k"], x["seq_lens"])[0]
    order = np.lexsort((np.arange(300), -sc))
    u, w = int(order[19]), int(order[40])
    x["k"][0, 0, w] = x["k"][0, 0, u]
    g_idx, _ = _run_decode(x, to_device(x), case, 20, [(0, 0)], "dup-row")
    kept = set(g_idx[0].tolist())
    assert min(u, w) in kept and max(u, w) not in kept


def test_zero_length_row():
    case = synth.small_case(B=2, h_q=4, h_k=1, h_v=2, d=64, S_max=64, N=8, dtype="bf16",
                            seed=61)
    lens = np.array([0, 64], np.int32)
    x = synth.make_inputs(case, lens)
    dx = to_device(x)
    idx = torch.empty((2, 4, 8), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 8, idx_out=idx)
    outd = saga.dense_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"])
    assert (idx[0].cpu() == -1).all()
    assert (out[0].cpu() == 0).all() and (outd[0].cpu() == 0).all()
    assert torch.isfinite(out).all()


def test_deterministic_and_workspace_reuse():
    case = synth.CASES["llama32_1b_8to4"]
    x = synth.make_inputs(case)
    dx = to_device(x)
    ws = saga.new_workspace(saga.workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 512)
                            + 4096, "cuda")
    ws.fill_(0xAB)   # contents left by someone else must not matter
    outs, idxs = [], []
    for _ in range(2):
        idx = torch.empty((case.B, case.h_q, 512), dtype=torch.int32, device="cuda")
        outs.append(saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 512,
                                     workspace=ws, idx_out=idx).cpu())
        idxs.append(idx.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(idxs[0], idxs[1])
    small = synth.small_case(B=1, h_q=4, h_k=1, h_v=2, d=64, S_max=200, N=10, seed=3)
    xs = synth.make_inputs(small)
    _run_decode(xs, to_device(xs), small, 10, all_pairs(1, 4), "after-reuse")


def test_timed_entry_matches_plain_entry():
    case = synth.CASES["llama32_1b_8to4"]
    x = synth.make_inputs(case)
    dx = to_device(x)
    B, h_q, h_k, h_v, d, S, N = case.B, case.h_q, case.h_k, case.h_v, case.d, case.S_max, case.N
    _say(f"[timed] B={B} h_q={h_q} h_k={h_k} h_v={h_v} d={d} S={S} N={N}")
    st = torch.cuda.current_stream()
    wsb = saga.saga_workspace_size(B, h_q, h_k, h_v, d, N, S, saga.SAGA_BF16)
    ws = saga.new_workspace(wsb, "cuda")
    res = []
    for nev in (0, 2, 4):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
        for e_ in evs:
            e_.record(st)
        out = torch.empty((B, h_q, d), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, h_q, N), dtype=torch.int32, device="cuda")
        rc = saga.saga_decode_attn_timed(dx["q"], dx["k"], dx["v"], dx["seq_lens"], out, B, h_q,
                                         h_k, h_v, d, N, st.cuda_stream, S, saga.SAGA_BF16, ws,
                                         wsb, idx, [e_.cuda_event for e_ in evs])
        assert rc == saga.SAGA_OK
        torch.cuda.synchronize()
        for a, b_ in zip(evs, evs[1:]):
            assert a.elapsed_time(b_) >= 0.0
        res.append((out.cpu(), idx.cpu()))
    plain = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], N).cpu()
    for o, i in res:
        assert torch.equal(o, plain) and torch.equal(i, res[0][1])


def test_kscan_scores_match_oracle_logits():
    for (dt, d) in (("f32", 64), ("bf16", 128), ("f32", 128), ("bf16", 64)):
        case = synth.small_case(B=2, h_q=12, h_k=3, h_v=3, d=d, S_max=1001, N=1, dtype=dt,
                                ragged=True, seed=67)
        x = synth.make_inputs(case)
        dx = to_device(x)
        sc = saga.debug_scores(dx["q"], dx["k"], dx["seq_lens"]).reshape(-1, 1001).cpu().numpy()
        ref = oracle.logits(x["q"], x["k"], x["seq_lens"])
        qa = np.abs(synth.as_f32(x["q"]).astype(np.float64))
        ka = np.abs(synth.as_f32(x["k"]).astype(np.float64))
        g = 12 // 3
        for r in range(24):
            b, i = divmod(r, 12)
            L = int(x["seq_lens"][b])
            # fp32 accumulation bound: (d + 2) u sum_c |q_c k_c| / sqrt(d), u = 2^-24
            mag = (ka[b, i // g, :L] @ qa[b, i]) / np.sqrt(d)
            bound = (d + 2) * 2.0 ** -24 * mag + 1e-30
            err = np.abs(sc[r, :L] - ref[r, :L])
            assert (err <= bound).all(), (dt, d, r, float((err / bound).max()))
            assert np.isnan(sc[r, L:]).all()


def _fallback_flags(dx, ws, case, N):
    flags = np.zeros(case.B * case.h_q, dtype=np.int32)
    st = saga.saga_debug_fallback_rows(ws, ws.numel(), case.B, case.h_q, case.h_k, case.h_v,
                                       case.d, N, case.S_max,
                                       saga.SAGA_F32 if case.dtype == "f32" else saga.SAGA_BF16,
                                       flags, torch.cuda.current_stream().cuda_stream)
    assert st == saga.SAGA_OK
    return flags


def test_clustered_top_entries_take_exact_fallback():
    # Batch row 0: the 300 largest logits of every head sit in the first chunk of
    # 1024 positions, more than that chunk's candidate list can carry, so the
    # selector cannot prove the union exact and must recompute those heads.
    case = synth.small_case(B=2, h_q=4, h_k=1, h_v=2, d=64, S_max=8192, N=300, dtype="bf16",
                            seed=71)
    x = synth.make_inputs(case)
    qsum = synth.as_f32(x["q"][0]).astype(np.float64).sum(axis=0)
    rng = np.random.default_rng(3)
    # logits spread geometrically over ~10 half-octave bins, so the bin of the
    # chunk's M-th key cannot hold all 300 of them
    alpha = 3.0 * 2.0 ** (np.arange(300) / 60.0)
    rows = alpha[:, None] * qsum[None, :] / np.linalg.norm(qsum) * 8.0 + rng.standard_normal((300, 64))
    x["k"][0, 0, :300] = synth.f32_to_bf16_bits(rows.astype(np.float32))
    dx = to_device(x)
    ws = saga.new_workspace(saga.workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 300),
                            "cuda")
    idx = torch.empty((2, 4, 300), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], 300, workspace=ws,
                           idx_out=idx)
    torch.cuda.synchronize()
    flags = _fallback_flags(dx, ws, case, 300)
    _say(f"    fallback flags {flags.tolist()}")
    pairs = all_pairs(2, 4)
    ref = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], 300, pairs=pairs)
    g_idx = idx.reshape(-1, 300).cpu().numpy()
    check_index_sets(g_idx, ref, x, pairs, 300)
    check_outputs(out.reshape(-1, 64).cpu().numpy(), g_idx, x, pairs, 2e-3)
    assert set(g_idx[0].tolist()) == set(range(300))
    # row 0's heads recompute their first chunk only (2); row 1 settles from the lists (0)
    assert flags[:4].tolist() == [2, 2, 2, 2] and flags[4:].tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("name", list(synth.CONCENTRATED))
def test_concentrated_attention(name):
    # sinks and a recency window: a large share of each head's top-N sits in the
    # last chunk, beyond what a list of M entries carries. The K-scan extends
    # such a chunk's list down to the lowest cutoff of the row's earlier chunks
    # in the same workgroup, so heads settle from the lists (flag 0); where the
    # window's chunks have no earlier chunk of the row in their workgroup, a
    # head recomputes those chunks only (flag 2). Never the whole row (flag 1).
    case = synth.CONCENTRATED[name]
    x = synth.make_inputs(case)
    dx = to_device(x)
    ws = saga.new_workspace(saga.workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"],
                                                case.N), "cuda")
    _say(f"[concentrated] {name}")
    idx = torch.empty((case.B, case.h_q, case.N), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], case.N, workspace=ws,
                           idx_out=idx)
    torch.cuda.synchronize()
    flags = _fallback_flags(dx, ws, case, case.N)
    pairs = all_pairs(case.B, case.h_q)
    ref = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], case.N, pairs=pairs)
    g_idx = idx.reshape(-1, case.N).cpu().numpy()
    nbad, ndiff = check_index_sets(g_idx, ref, x, pairs, case.N)
    err = check_outputs(out.reshape(-1, case.d).cpu().numpy(), g_idx, x, pairs,
                        tol_for(case.dtype))
    counts = np.bincount(flags, minlength=3)
    _say(f"    rows={len(pairs)} differing-rows={nbad} sym-diff={ndiff} max|err|={err:.2e} "
         f"settled={counts[0]} chunk-recompute={counts[2]} full-recompute={counts[1]}")
    assert counts[1] == 0


@pytest.mark.parametrize("B", [4, 1])
def test_concentrated_attention_small_batch(B):
    # the same sink and recency structure at batch sizes whose K-scan items are
    # 512 (B = 4) or 256 (B = 1) positions, one item per workgroup: the window's
    # chunks have no earlier chunk of their row to lend a floor, so heads may
    # recompute chunks (flag 2), but the kept sets and outputs match the oracle
    from dataclasses import replace
    case = replace(synth.CASES["qwen25_1p5b_b64_32k"], B=B, name=f"recency_b{B}",
                   structure="recency_sink")
    x = synth.make_inputs(case)
    dx = to_device(x)
    _say(f"[concentrated] small batch B={B}")
    ws = saga.new_workspace(saga.workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"],
                                                case.N), "cuda")
    idx = torch.empty((case.B, case.h_q, case.N), dtype=torch.int32, device="cuda")
    out = saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], case.N, workspace=ws,
                           idx_out=idx)
    torch.cuda.synchronize()
    flags = _fallback_flags(dx, ws, case, case.N)
    pairs = all_pairs(case.B, case.h_q)
    ref = oracle.topn_attn(x["q"], x["k"], x["v"], x["seq_lens"], case.N, pairs=pairs)
    g_idx = idx.reshape(-1, case.N).cpu().numpy()
    nbad, ndiff = check_index_sets(g_idx, ref, x, pairs, case.N)
    err = check_outputs(out.reshape(-1, case.d).cpu().numpy(), g_idx, x, pairs,
                        tol_for(case.dtype))
    counts = np.bincount(flags, minlength=3)
    _say(f"    differing-rows={nbad} sym-diff={ndiff} max|err|={err:.2e} "
         f"settled={counts[0]} chunk-recompute={counts[2]} full-recompute={counts[1]}")
    assert counts[1] == 0


def test_workloads_report_fallback_rows():
    for name in ("llama32_1b_8to4", "qwen25_1p5b_2to1_ragged", "qwen25_1p5b_b64_32k"):
        case = synth.CASES[name]
        x = synth.make_inputs(case)
        dx = to_device(x)
        ws = saga.new_workspace(saga.workspace_size(dx["q"], dx["k"], dx["v"], dx["seq_lens"],
                                                    case.N), "cuda")
        saga.decode_attn(dx["q"], dx["k"], dx["v"], dx["seq_lens"], case.N, workspace=ws)
        flags = _fallback_flags(dx, ws, case, case.N)
        _say(f"    {name}: {int(flags.sum())} of {flags.size} heads took the dense fallback")
        assert flags.sum() <= flags.size // 20
        del dx, ws
        torch.cuda.empty_cache()
