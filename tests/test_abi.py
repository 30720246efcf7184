"""C-ABI checks that need no GPU.

libsaga.so must load without a device, export every function include/saga.h
declares, and reject every invalid scalar argument with its status code on
the host, before any HIP call (so these run on a machine with no GPU).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saga.h")

saga = pytest.importorskip("sparse_asymmetric_gqa_amd")

FAKE = 0x10000   # a 16-byte-aligned non-null "device pointer" never dereferenced here


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(saga_[a-z_]+)\s*\(", text)))


def test_exports_match_header():
    declared = _declared_functions()
    assert set(declared) == set(saga.EXPORTS)
    lib = ctypes.CDLL(saga.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = saga.status_string(code)
        assert s and s != "unknown status"
    assert saga.status_string(7) == "unknown status"


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, h_q=8, h_k=2, h_v=4, d=64, N=16,
             stream=None, S=100, dt=saga.SAGA_BF16, ws=FAKE * 16, wsb=1 << 40, idx=None)
    a.update(kw)
    return saga.saga_decode_attn(a["q"], a["k"], a["v"], a["lens"], a["out"], a["B"], a["h_q"],
                                 a["h_k"], a["h_v"], a["d"], a["N"], a["stream"], a["S"], a["dt"],
                                 a["ws"], a["wsb"], a["idx"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(k=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(v=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(lens=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(out=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(B=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(h_q=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(N=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(S=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(h_q=9), saga.SAGA_ERR_INVALID_ARG),          # 9 % 2 != 0
    (dict(h_v=3), saga.SAGA_ERR_INVALID_ARG),          # 8 % 3 != 0
    (dict(h_k=8, h_v=4), saga.SAGA_ERR_INVALID_ARG),   # h_k > h_v
    (dict(dt=5), saga.SAGA_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), saga.SAGA_ERR_INVALID_ARG),     # misaligned
    (dict(d=96), saga.SAGA_ERR_UNSUPPORTED),
    (dict(d=256), saga.SAGA_ERR_UNSUPPORTED),
    (dict(h_q=128, h_k=1, h_v=128), saga.SAGA_ERR_UNSUPPORTED),   # key group of 128
    (dict(ws=None), saga.SAGA_ERR_WORKSPACE),
    (dict(wsb=1024), saga.SAGA_ERR_WORKSPACE),
    (dict(ws=FAKE * 16 + 16), saga.SAGA_ERR_WORKSPACE),  # not 256-byte aligned
])
def test_decode_rejects_bad_arguments_on_host(kw, code):
    assert _decode(**kw) == code


def test_dense_and_debug_reject_bad_arguments_on_host():
    d = saga.saga_dense_attn
    ok = dict(B=2, h_q=8, h_k=2, h_v=4, d=64, S=100)
    assert d(None, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 4, 64, None, 100, 1, FAKE * 16, 1 << 40) == -1
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 4, 2, 64, None, 100, 1, FAKE * 16, 1 << 40) == -1
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 4, 80, None, 100, 1, FAKE * 16, 1 << 40) == -2
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 4, 64, None, 100, 1, FAKE * 16, 64) == -3
    s = saga.saga_debug_scores
    assert s(FAKE, FAKE, FAKE, None, 2, 8, 2, 64, None, 100, 1) == -1
    assert s(FAKE, FAKE, FAKE, FAKE, 2, 8, 3, 64, None, 100, 1) == -1
    assert s(FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 32, None, 100, 1) == -2
    assert ok


def test_workspace_sizes():
    ws = saga.saga_workspace_size
    assert ws(2, 8, 2, 4, 64, 16, 100, 1) > 0
    assert ws(2, 8, 2, 4, 64, 0, 100, 1) == 0
    assert ws(2, 8, 2, 4, 48, 16, 100, 1) == 0
    assert ws(2, 8, 4, 2, 64, 16, 100, 1) == 0
    for args in [(1, 4, 1, 2, 64, 64, 1024, 0), (64, 12, 1, 2, 128, 1024, 32768, 1),
                 (8, 32, 4, 8, 64, 512, 8192, 1), (3, 6, 2, 2, 128, 7, 33, 1)]:
        n = ws(*args)
        assert n % 256 == 0
        B, h_q, _, _, d, N, S, _ = args
        # at least the fp32 logit rows, the kept lists and one partial per row
        assert n >= B * h_q * (4 * S + 8 * N + 4 * (d + 2))
        # growing any size never shrinks the workspace
        assert ws(B, h_q, args[2], args[3], d, N + 300, S, 1) >= n
        assert ws(B, h_q, args[2], args[3], d, N, S + 5000, 1) >= n
    dw = saga.saga_dense_workspace_size
    # one (m, l, acc[d]) partial per row and chunk: 1024 positions where that
    # still gives 128 (b, key head, chunk) items, else 512 or 256 (key groups
    # of up to 16 heads); 256 positions for wider key groups
    assert dw(64, 12, 2, 2, 128, 32768, 1) >= 64 * 12 * 32 * 130 * 4
    assert dw(1, 12, 2, 2, 128, 32768, 1) >= 12 * 64 * 130 * 4      # 512: 128 items
    assert dw(1, 12, 1, 2, 128, 8192, 1) >= 12 * 32 * 130 * 4       # 256: 32 items
    assert dw(1, 64, 1, 2, 64, 1000, 1) >= 64 * 4 * 66 * 4
    assert dw(1, 4, 1, 2, 64, 1025, 0) >= dw(1, 4, 1, 2, 64, 1000, 0)
    assert dw(1, 4, 1, 2, 72, 10, 1) == 0


def test_timed_entry_rejects_bad_event_lists_on_host():
    t = saga.saga_decode_attn_timed
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 4, 64, 16, None, 100, saga.SAGA_BF16,
            FAKE * 16, 1 << 40, None)
    assert t(*args, [FAKE] * 5) == saga.SAGA_ERR_INVALID_ARG      # more than four boundaries
    assert t(*args, [FAKE, 0]) == saga.SAGA_ERR_INVALID_ARG       # a null event
    bad = list(args)
    bad[5] = 0                                                   # B = 0, checked before events
    assert t(*bad, []) == saga.SAGA_ERR_INVALID_ARG


def _atopn(fn, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, h_q=8, h_k=2, h_v=4, d=64, N=16,
             stream=None, S=100, dt=saga.SAGA_BF16, ws=FAKE * 16, wsb=1 << 40, tau=FAKE)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["lens"], a["out"], a["B"], a["h_q"], a["h_k"], a["h_v"],
            a["d"], a["N"], a["stream"], a["S"], a["dt"], a["ws"], a["wsb"], a["tau"])
    return fn(*args)


@pytest.mark.parametrize("fn", ["saga_atopn_calibrate", "saga_atopn_attn"])
@pytest.mark.parametrize("kw,code", [
    (dict(tau=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(q=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(out=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(N=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(h_k=8, h_v=4), saga.SAGA_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), saga.SAGA_ERR_INVALID_ARG),
    (dict(d=96), saga.SAGA_ERR_UNSUPPORTED),
    (dict(h_q=64, h_k=2, h_v=4), saga.SAGA_ERR_UNSUPPORTED),     # key group of 32
    (dict(S=600000), saga.SAGA_ERR_UNSUPPORTED),                  # > 512 chunks
    (dict(ws=None), saga.SAGA_ERR_WORKSPACE),
    (dict(wsb=1024), saga.SAGA_ERR_WORKSPACE),
])
def test_atopn_rejects_bad_arguments_on_host(fn, kw, code):
    assert _atopn(getattr(saga, fn), **kw) == code


def test_atopn_workspace_holds_2N_slots():
    aw, ws = saga.saga_atopn_workspace_size, saga.saga_workspace_size
    for args in [(64, 12, 1, 2, 128, 1024, 32768, 1), (3, 6, 2, 2, 128, 7, 33, 1)]:
        B, h_q, h_k, h_v, d, N, S, dt = args
        n = aw(*args)
        # the kept lists of 2N slots (index + logit) per row, beyond the decode
        # workspace's N-slot lists
        assert n % 256 == 0 and n >= B * h_q * 2 * N * 8
        n1 = aw(B, h_q, h_k, h_v, d, N + 64, S, dt)
        assert n1 - n >= B * h_q * 2 * 64 * 8 - 4 * 256
    assert aw(1, 4, 1, 2, 72, 10, 100, 1) == 0 and aw(1, 4, 1, 2, 64, 0, 100, 1) == 0


def _sparq(**kw):
    a = dict(q=FAKE, k=FAKE, kt=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, h_q=8, h_k=2, h_v=4, d=64,
             N=16, r=8, local=4, vm=None, stream=None, S=104, dt=saga.SAGA_BF16, ws=FAKE * 16,
             wsb=1 << 40)
    a.update(kw)
    return saga.saga_sparq_attn(a["q"], a["k"], a["kt"], a["v"], a["lens"], a["out"], a["B"],
                                a["h_q"], a["h_k"], a["h_v"], a["d"], a["N"], a["r"], a["local"],
                                a["vm"], a["stream"], a["S"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,code", [
    (dict(kt=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(q=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(v=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(out=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(r=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(r=65), saga.SAGA_ERR_INVALID_ARG),           # r > d
    (dict(local=-1), saga.SAGA_ERR_INVALID_ARG),
    (dict(local=17), saga.SAGA_ERR_INVALID_ARG),       # local > N
    (dict(N=0, local=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(kt=FAKE + 8), saga.SAGA_ERR_INVALID_ARG),    # misaligned
    (dict(vm=FAKE + 2), saga.SAGA_ERR_INVALID_ARG),    # v_mean not 4-byte aligned
    (dict(h_k=8, h_v=4), saga.SAGA_ERR_INVALID_ARG),
    (dict(d=96, r=8), saga.SAGA_ERR_UNSUPPORTED),
    (dict(h_q=64, h_k=2, h_v=4), saga.SAGA_ERR_UNSUPPORTED),     # key group of 32
    (dict(S=600000), saga.SAGA_ERR_UNSUPPORTED),                  # > 512 chunks
    (dict(N=5000, local=0), saga.SAGA_ERR_UNSUPPORTED),           # kept list beyond LDS staging
    (dict(S=100), saga.SAGA_ERR_UNSUPPORTED),                     # bf16 rows not 16-byte pieces
    (dict(S=102, dt=saga.SAGA_F32), saga.SAGA_ERR_UNSUPPORTED),
    (dict(ws=None), saga.SAGA_ERR_WORKSPACE),
    (dict(wsb=1024), saga.SAGA_ERR_WORKSPACE),
    (dict(ws=FAKE * 16 + 16), saga.SAGA_ERR_WORKSPACE),
])
def test_sparq_rejects_bad_arguments_on_host(kw, code):
    assert _sparq(**kw) == code


def test_sparq_workspace_extends_the_decode_workspace():
    sw, ws = saga.saga_sparq_workspace_size, saga.saga_workspace_size
    for B, h_q, h_k, h_v, d, N, S, dt in [(64, 12, 1, 2, 128, 1024, 32768, 1),
                                          (3, 6, 2, 2, 64, 7, 40, 0)]:
        n = sw(B, h_q, h_k, h_v, d, N, 16, S, dt)
        base = ws(B, h_q, h_k, h_v, d, N, S, dt)
        assert n % 256 == 0 and n > base
        # dims, the scan operand, 1/tau and q/tau: bounded by their largest sizes
        e = 2 if dt == 1 else 4
        extra = B * h_k * d * 4 + B * h_k * (d // 16) * 64 * 4 * e + B * h_q * 4 + B * h_q * d * 4
        if B * h_k * (S // 1024) >= 256:
            # same 1024-position items and no split gather as the decode workspace
            assert n <= base + extra + 4 * 256
        else:
            # the scan keeps 1024-position items where the decode call uses 256
            assert n <= base + extra + B * h_q * -(-S // 1024) * 1024 * 8 + 8 * 256
    assert sw(1, 4, 1, 2, 64, 10, 0, 100, 1) == 0 and sw(1, 4, 1, 2, 64, 10, 65, 100, 1) == 0


def _merge(**kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, L=700, D=512, h_q=8, h_kt=4, d=64, strat=0,
             dt=saga.SAGA_BF16, merged=FAKE, sigma=FAKE, pw=None, obj=None, stats=None,
             ws=FAKE * 16, wsb=1 << 40)
    a.update(kw)
    return saga.saga_key_merge(a["x"], a["wq"], a["wk"], a["L"], a["D"], a["h_q"], a["h_kt"],
                               a["d"], a["strat"], a["dt"], a["merged"], a["sigma"], a["pw"],
                               a["obj"], a["stats"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(wk=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(merged=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(sigma=None), saga.SAGA_ERR_INVALID_ARG),
    (dict(strat=3), saga.SAGA_ERR_INVALID_ARG),
    (dict(h_kt=3, h_q=6), saga.SAGA_ERR_INVALID_ARG),     # odd teacher key-head count
    (dict(h_q=6), saga.SAGA_ERR_INVALID_ARG),             # h_q not a multiple of h_kt
    (dict(L=0), saga.SAGA_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), saga.SAGA_ERR_INVALID_ARG),        # misaligned
    (dict(dt=saga.SAGA_F32), saga.SAGA_ERR_UNSUPPORTED),
    (dict(d=144, h_q=8), saga.SAGA_ERR_UNSUPPORTED),      # beyond the LDS Jacobi matrix
    (dict(d=40), saga.SAGA_ERR_UNSUPPORTED),              # not a multiple of 16
    (dict(D=500), saga.SAGA_ERR_UNSUPPORTED),
    (dict(h_kt=26, h_q=26), saga.SAGA_ERR_UNSUPPORTED),   # beyond the subset DP
    (dict(ws=None), saga.SAGA_ERR_WORKSPACE),
    (dict(wsb=4096), saga.SAGA_ERR_WORKSPACE),
])
def test_key_merge_rejects_bad_arguments_on_host(kw, code):
    assert _merge(**kw) == code


def test_key_merge_timed_and_permute_reject_on_host():
    tm = saga.saga_key_merge_timed
    args = (FAKE, FAKE, FAKE, 700, 512, 8, 4, 64, 0, saga.SAGA_BF16, FAKE, FAKE, None, None, None,
            FAKE * 16, 1 << 40, None)
    assert tm(*args, None, 1) == saga.SAGA_ERR_INVALID_ARG
    assert tm(*args, None, 6) == saga.SAGA_ERR_INVALID_ARG
    pm = saga.saga_merge_permute
    ok = (FAKE, FAKE, FAKE, FAKE, 512, 8, 4, 64, saga.SAGA_BF16, FAKE * 2, FAKE * 3, FAKE * 4,
          None)
    assert pm(None, *ok[1:]) == saga.SAGA_ERR_INVALID_ARG
    assert pm(*ok[:4], 512, 6, 4, 64, *ok[8:]) == saga.SAGA_ERR_INVALID_ARG      # h_q % h_kt
    assert pm(*ok[:4], 512, 8, 4, 60, *ok[8:]) == saga.SAGA_ERR_UNSUPPORTED      # 120-byte blocks
    assert pm(*ok[:4], 512, 8, 4, 64, 7, *ok[9:]) == saga.SAGA_ERR_INVALID_ARG   # dtype
    assert pm(*ok[:9], FAKE * 2 + 8, *ok[10:]) == saga.SAGA_ERR_INVALID_ARG     # misaligned


def test_key_merge_workspace_size():
    mw = saga.saga_key_merge_workspace_size
    assert mw(700, 512, 8, 4, 64) > 0 and mw(700, 512, 8, 4, 64) % 256 == 0
    # one 256 x 256 fp32 X^T X partial per (tile, split), then C, W C, the
    # statistics, the rotation records and the per-pair matrices
    n = mw(131072, 2048, 32, 8, 64)
    assert 36 * 7 * 256 * 256 * 4 < n < 36 * 7 * 256 * 256 * 4 + (96 << 20)
    assert mw(700, 512, 8, 3, 64) == 0 and mw(700, 512, 8, 4, 136) == 0 and mw(0, 512, 8, 4, 64) == 0


def test_noalloc_entry_checks_on_host():
    """The no-allocation entry: its static scratch size, and every argument
    check (including the scratch bound) decided on the host before any HIP call."""
    assert saga.saga_noalloc_scratch_bytes() == 128 << 20
    f = saga.saga_decode_attn_noalloc
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 4, 64, 16, None, 100, saga.SAGA_BF16, None]

    def call(**kw):
        a = list(base)
        for k_, v_ in kw.items():
            a[int(k_[1:])] = v_
        return f(*a)
    assert call(a0=None) == saga.SAGA_ERR_INVALID_ARG       # q
    assert call(a4=None) == saga.SAGA_ERR_INVALID_ARG       # out
    assert call(a10=0) == saga.SAGA_ERR_INVALID_ARG         # N
    assert call(a7=4, a8=2) == saga.SAGA_ERR_INVALID_ARG    # h_k > h_v
    assert call(a9=96) == saga.SAGA_ERR_UNSUPPORTED         # d
    # a shape whose decode workspace exceeds the static buffer
    big = saga.saga_workspace_size(64, 12, 1, 2, 128, 1024, 1 << 20, saga.SAGA_BF16)
    assert big > saga.saga_noalloc_scratch_bytes()
    assert call(a5=64, a6=12, a7=1, a8=2, a9=128, a10=1024, a12=1 << 20) == \
        saga.SAGA_ERR_TOO_LARGE


def test_dense_chunk_rule():
    # The dense workspace holds B h_q (d + 2) floats per chunk of the row, so
    # its size gives the chunk count the library picked. The rule: among the
    # chunk lengths 1024, 512 and 256 that leave at most 128 chunks per row,
    # the longest giving at least 256 (b, key head, chunk) items, else the
    # shortest of them (1024 when even that leaves more than 128); key groups
    # wider than 16 always take 256.
    dw = saga.saga_dense_workspace_size

    def expected(B, h_k, S, g):
        if g > 16:
            return 256
        shortest = 1024
        for C in (1024, 512, 256):
            parts = -(-S // C)
            if parts > 128:
                break
            if B * h_k * parts >= 256:
                return C
            shortest = C
        return shortest

    rng = __import__("random").Random(5)
    shapes = [(1, 12, 1, 2, 8192), (1, 12, 2, 2, 32768), (16, 12, 1, 2, 8192),
              (64, 12, 2, 2, 32768), (1, 12, 1, 2, 131072), (2, 64, 1, 2, 5000)]
    for _ in range(60):
        h_k = rng.choice([1, 2, 4])
        g = rng.choice([1, 2, 4, 8, 16, 32])
        shapes.append((rng.choice([1, 2, 3, 4, 8, 16, 64]), h_k * g, h_k,
                       h_k * rng.choice([1, 2]), rng.randint(1, 140000)))
    for B, h_q, h_k, h_v, S in shapes:
        if h_q % h_v or h_q // h_v > 64:
            continue
        d = 128
        n = dw(B, h_q, h_k, h_v, d, S, 1)
        C = expected(B, h_k, S, h_q // h_k)
        need = B * h_q * (-(-S // C)) * (d + 2) * 4
        # the partials are the dense workspace's only area (256-byte aligned)
        assert n == (need + 255) // 256 * 256, (B, h_q, h_k, h_v, S, C, n, need)
