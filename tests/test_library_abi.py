"""The C-ABI library: it loads, exports every symbol the header declares, and
rejects bad arguments on the host before any HIP call (CPU only: every call
here fails validation, so no kernel is launched and no device is touched)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from structured_sparse_causal_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

SA_OK, INVALID, UNSUPPORTED, HIP, WORKSPACE = 0, -1, -2, -3, -4
PI, WINDOW, ECP = 0, 1, 2
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), "missing export " + n
    assert set(names) == set(binding.EXPORTED)


def test_version_and_status_strings(lib):
    assert lib.sparse_attn_version() == 101
    assert lib.sparse_attn_status_string(SA_OK) == b"ok"
    assert lib.sparse_attn_status_string(WORKSPACE) == b"workspace too small"
    assert lib.sparse_attn_status_string(12345) == b"unknown status"


# Fake, never-dereferenced device addresses (validation fails before use).
Q, K, V, A, O, WS = (0x100000 * (i + 1) for i in range(6))


def fwd(lib, q=Q, k=K, v=V, a=A, o=O, B=1, Hq=2, Hkv=2, N=256, d=64, dtype=BF16, mode=PI,
        k_win=32, pi=64, M=3, seg=0, ws=None, wsb=0):
    return lib.sparse_attn_fwd(q, k, v, a, o, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg,
                               ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
    (dict(mode=9), INVALID), (dict(k_win=-1), INVALID), (dict(M=-1), INVALID),
    (dict(pi=0), INVALID), (dict(mode=ECP, seg=0), INVALID), (dict(q=None), INVALID),
    (dict(o=None), INVALID), (dict(a=None), INVALID), (dict(q=Q + 8), INVALID),
    (dict(a=A + 2), INVALID), (dict(o=Q), INVALID), (dict(o=K + 64), INVALID),
    (dict(), WORKSPACE), (dict(ws=WS, wsb=16), WORKSPACE),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code
    assert lib.sparse_attn_last_error() != b""


def test_fwd_alpha_optional_without_skips(lib):
    # WINDOW and ECP ignore alpha; validation must not demand it.  Use an
    # overlapping output so the call still fails before any launch.
    assert fwd(lib, a=None, mode=WINDOW, o=Q) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()
    assert fwd(lib, a=None, mode=ECP, seg=64, o=Q) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()


def test_fwd_workspace_sizes(lib):
    ws = lib.sparse_attn_fwd_workspace_size
    # pi-Attention with skip keys: per row an (m, l) fp32 pair and a d-wide
    # accumulator in the I/O dtype, for one chunk of (batch, head) slices: at
    # most 128 MiB, split into balanced chunks.
    rows = 32 * 16384                                   # 71.3 MB: one chunk
    r256 = lambda x: -(-x // 256) * 256
    assert ws(2, 16, 16, 16384, 64, BF16, PI, 256, 1024, 15, 0) == r256(rows * 8) + r256(rows * 64 * 2)
    assert ws(1, 2, 2, 100, 64, F32, PI, 32, 64, 3, 0) == r256(2 * 100 * 8) + r256(2 * 100 * 64 * 4)
    # 64 slices of 4.3 MB (fp32, d = 128, N = 8192) -> 3 chunks of 22 slices.
    rows = 22 * 8192
    assert ws(4, 16, 16, 8192, 128, F32, PI, 256, 1024, 15, 0) == r256(rows * 8) + r256(rows * 128 * 4)
    assert ws(1, 32, 32, 65536, 128, BF16, WINDOW, 1024, 0, 0, 0) == 0
    assert ws(4, 12, 12, 4096, 64, BF16, ECP, 0, 0, 0, 512) == 0
    assert ws(1, 2, 2, 256, 64, F32, PI, 32, 64, 0, 0) == 0          # M = 0
    assert ws(1, 2, 2, 256, 64, F32, PI, 300, 64, 4, 0) == 0         # every skip inside the window
    assert ws(1, 2, 2, 100, 64, F32, PI, 32, 64, 3, 0) > 0           # position 64 has key 0
    assert ws(1, 2, 2, 64, 64, F32, PI, 32, 64, 3, 0) == 0           # no position reaches a skip
    assert ws(1, 2, 2, 256, 96, F32, PI, 32, 64, 3, 0) == 0          # rejected arguments


def dec(lib, q=Q, kc=K, vc=V, lens=A, a=A + 4096, o=O, B=2, Hq=8, Hkv=2, L=512, d=128, dtype=BF16,
        mode=PI, k_win=64, pi=64, M=3, seg=0, ws=WS, wsb=1 << 30):
    return lib.sparse_attn_decode(q, kc, vc, lens, a, o, B, Hq, Hkv, L, d, dtype, mode, k_win, pi, M,
                                  seg, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), UNSUPPORTED), (dict(Hq=6, Hkv=4), INVALID), (dict(L=0), INVALID),
    (dict(lens=None), INVALID), (dict(a=None), INVALID), (dict(mode=ECP, seg=-3), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE), (dict(ws=WS + 64), INVALID),
    (dict(o=K + 128), INVALID), (dict(o=WS), INVALID), (dict(lens=A + 2), INVALID),
])
def test_decode_rejects(lib, kw, code):
    assert dec(lib, **kw) == code


def test_decode_workspace_size(lib):
    ws = lib.sparse_attn_decode_workspace_size
    # 2048 window rows below the query -> 8 splits of 256, plus one split for the
    # query row and the skip keys.
    assert ws(64, 32, 8, 32768, 128, BF16, PI, 2048, 2048, 15, 0) == 64 * 32 * 9 * 132 * 4
    assert ws(64, 32, 8, 32768, 128, BF16, WINDOW, 2048, 0, 0, 0) == 64 * 32 * 9 * 132 * 4
    assert ws(1, 1, 1, 100, 64, F32, ECP, 0, 0, 0, 512) == 256 * ((1 * 1 * 2 * 68 * 4 + 255) // 256)
    assert ws(2, 2, 2, 300, 64, BF16, WINDOW, 0, 0, 0, 0) == 256 * ((2 * 2 * 1 * 68 * 4 + 255) // 256)  # k = 0
    assert ws(1, 1, 1, 100, 60, F32, ECP, 0, 0, 0, 512) == 0


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        binding.fwd(q, q, q, mode="window", k_win=2)
    qb = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError):   # the differentiable entry has no host path either
        binding.attention(qb, qb, qb, mode="window", k_win=2)


def fwd_lse(lib, lse=WS, **kw):
    p = dict(q=Q, k=K, v=V, a=A, o=O, B=1, Hq=2, Hkv=2, N=256, d=64, dtype=BF16, mode=WINDOW,
             k_win=32, pi=64, M=3, seg=0)
    p.update(kw)
    return lib.sparse_attn_fwd_lse(p["q"], p["k"], p["v"], p["a"], p["o"], lse, p["B"], p["Hq"], p["Hkv"],
                                   p["N"], p["d"], p["dtype"], p["mode"], p["k_win"], p["pi"], p["M"],
                                   p["seg"], None, 0, None)


def test_fwd_lse_rejects(lib):
    assert fwd_lse(lib, lse=None) == INVALID
    assert b"lse" in lib.sparse_attn_last_error()
    assert fwd_lse(lib, lse=WS + 2) == INVALID                     # misaligned
    assert fwd_lse(lib, lse=Q + 64) == INVALID                     # overlaps q
    assert b"lse overlaps" in lib.sparse_attn_last_error()
    assert fwd_lse(lib, d=96) == UNSUPPORTED


DO, DQ, DK, DV, DA, LSE = (0x10000000 * (i + 1) for i in range(6))


def bwd(lib, q=Q, k=K, v=V, a=A, o=O, lse=LSE, dO=DO, dq=DQ, dk=DK, dv=DV, da=DA, B=1, Hq=2, Hkv=2,
        N=256, d=64, dtype=BF16, mode=PI, k_win=32, pi=64, M=3, seg=0, ws=None, wsb=0):
    return lib.sparse_attn_bwd(q, k, v, a, o, lse, dO, dq, dk, dv, da, B, Hq, Hkv, N, d, dtype, mode,
                               k_win, pi, M, seg, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(Hq=3), INVALID),
    (dict(N=0), INVALID), (dict(mode=ECP, seg=0), INVALID), (dict(lse=None), INVALID),
    (dict(dO=None), INVALID), (dict(dk=None), INVALID), (dict(a=None), INVALID),
    (dict(da=None), INVALID), (dict(dq=DQ + 8), INVALID), (dict(lse=LSE + 1), INVALID),
    (dict(), WORKSPACE), (dict(ws=WS, wsb=64), WORKSPACE), (dict(ws=WS + 16, wsb=1 << 30), INVALID),
    (dict(dq=Q, ws=WS, wsb=1 << 30), INVALID), (dict(dk=DQ + 256, ws=WS, wsb=1 << 30), INVALID),
    (dict(da=LSE, ws=WS, wsb=1 << 30), INVALID), (dict(dv=WS + 1024, ws=WS, wsb=1 << 30), INVALID),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(lib, **kw) == code
    assert lib.sparse_attn_last_error() != b""


def test_bwd_dalpha_optional_without_gate(lib):
    # Window and ECP take no alpha and give no dalpha: validation passes them
    # and stops at the overlapping gradient.
    assert bwd(lib, a=None, da=None, mode=WINDOW, dq=Q, ws=WS, wsb=1 << 30) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()
    assert bwd(lib, a=None, da=None, mode=ECP, seg=64, dq=Q, ws=WS, wsb=1 << 30) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()


def test_bwd_workspace_sizes(lib):
    ws = lib.sparse_attn_bwd_workspace_size
    r256 = lambda x: -(-x // 256) * 256
    # Per query row D_i = dO_i . o_i and c_i (lse and log-gate term), each with a
    # 16-float tail; the skip-key contributions are added into dq, dk and dv in
    # place, so skip keys need no more.
    rows = 2 * 16 * 4096
    assert ws(2, 16, 16, 4096, 64, BF16, WINDOW, 256, 0, 0, 0) == 2 * r256((rows + 16) * 4)
    assert ws(2, 16, 16, 4096, 64, BF16, PI, 256, 1024, 3, 0) == 2 * r256((rows + 16) * 4)
    assert ws(1, 8, 2, 1000, 128, BF16, PI, 60, 70, 8, 0) == 2 * r256((8000 + 16) * 4)
    assert ws(1, 2, 2, 256, 64, BF16, PI, 300, 64, 4, 0) == 2 * r256((512 + 16) * 4)   # skips inside window
    assert ws(1, 2, 2, 256, 64, BF16, ECP, 0, 0, 0, 64) == 2 * r256((512 + 16) * 4)
    assert ws(1, 2, 2, 256, 64, F32, WINDOW, 8, 0, 0, 0) == 0                        # bf16 only
    assert ws(1, 2, 2, 256, 80, BF16, WINDOW, 8, 0, 0, 0) == 0


def ring(lib, q=Q, kr=K, vr=V, lens=A, a=A + 4096, o=O, B=2, Hq=8, Hkv=2, R=512, d=128, dtype=BF16,
         mode=PI, k_win=64, pi=64, M=3, seg=0, ws=WS, wsb=1 << 30):
    return lib.sparse_attn_decode_ring(q, kr, vr, lens, a, o, B, Hq, Hkv, R, d, dtype, mode, k_win, pi, M, seg,
                                       ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=F32), UNSUPPORTED), (dict(d=80), UNSUPPORTED), (dict(R=0), INVALID),
    (dict(R=192), INVALID),                        # M*pi + 1 = 193 rows must stay resident
    (dict(mode=WINDOW, k_win=600), INVALID),       # k_win + 1 = 601 > R
    (dict(mode=ECP, seg=300), INVALID),            # 2*seg = 600 > R
    (dict(lens=None), INVALID), (dict(a=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(o=K + 128), INVALID), (dict(ws=WS + 64), INVALID),
])
def test_decode_ring_rejects(lib, kw, code):
    assert ring(lib, **kw) == code


def test_decode_ring_accepts_minimal_span(lib):
    # R = M*pi + 1 exactly is valid: validation passes and stops at the
    # overlapping output.
    assert ring(lib, R=193, o=Q) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()


def test_decode_ring_workspace_size(lib):
    ws = lib.sparse_attn_decode_ring_workspace_size
    # planned like a contiguous cache of R rows
    assert ws(64, 32, 8, 30721, 128, BF16, PI, 2048, 2048, 15, 0) == \
        lib.sparse_attn_decode_workspace_size(64, 32, 8, 30721, 128, BF16, PI, 2048, 2048, 15, 0) > 0
    assert ws(64, 32, 8, 30720, 128, BF16, PI, 2048, 2048, 15, 0) == 0      # ring too short
    assert ws(2, 8, 2, 512, 128, F32, WINDOW, 64, 0, 0, 0) == 0             # bf16 only


TAB = 0x30000000


def paged(lib, q=Q, kp=K, vp=V, tab=TAB, lens=A, a=A + 4096, o=O, B=2, Hq=8, Hkv=2, num_pages=64, P=64,
          max_pages=16, d=128, dtype=BF16, mode=PI, k_win=64, pi=64, M=3, seg=0, ws=WS, wsb=1 << 30):
    return lib.sparse_attn_decode_paged(q, kp, vp, tab, lens, a, o, B, Hq, Hkv, num_pages, P, max_pages, d, dtype,
                                        mode, k_win, pi, M, seg, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=F32), UNSUPPORTED), (dict(d=96), UNSUPPORTED), (dict(P=48), INVALID), (dict(P=4), INVALID),
    (dict(P=8192), INVALID), (dict(max_pages=0), INVALID), (dict(num_pages=0), INVALID),
    (dict(M=64), UNSUPPORTED), (dict(tab=None), INVALID), (dict(tab=TAB + 2), INVALID),
    (dict(o=TAB), INVALID), (dict(ws=None), WORKSPACE), (dict(Hq=6, Hkv=4), INVALID),
    (dict(num_pages=1 << 20, Hkv=64, Hq=64), INVALID),
])
def test_decode_paged_rejects(lib, kw, code):
    assert paged(lib, **kw) == code


def test_decode_paged_workspace_size(lib):
    ws = lib.sparse_attn_decode_paged_workspace_size
    # planned like a contiguous cache of max_pages * page_size rows
    assert ws(64, 32, 8, 64, 512, 128, BF16, PI, 2048, 2048, 15, 0) == \
        lib.sparse_attn_decode_workspace_size(64, 32, 8, 32768, 128, BF16, PI, 2048, 2048, 15, 0)
    assert ws(1, 1, 1, 48, 4, 64, BF16, WINDOW, 8, 0, 0, 0) == 0           # page size not a power of two
    assert ws(1, 1, 1, 64, 4, 64, F32, WINDOW, 8, 0, 0, 0) == 0


WINDOW_BIDIR, SSPLIT, ECP_FULL = 3, 4, 5


def test_further_mask_modes_validation(lib):
    # segment modes need seg >= 1; the two-sided window needs k_win >= 0
    assert fwd(lib, mode=SSPLIT, seg=0) == INVALID
    assert fwd(lib, mode=ECP_FULL, seg=0) == INVALID
    assert fwd(lib, mode=WINDOW_BIDIR, k_win=-1) == INVALID
    for m, kw in ((WINDOW_BIDIR, dict(k_win=8)), (SSPLIT, dict(seg=64)), (ECP_FULL, dict(seg=64))):
        assert fwd(lib, mode=m, a=None, o=Q, **kw) == INVALID            # valid up to the overlap
        assert b"overlaps" in lib.sparse_attn_last_error()
        assert lib.sparse_attn_fwd_workspace_size(1, 2, 2, 256, 64, BF16, m, 8, 0, 0, 64) == 0
    # a decoded token has no later keys: the two non-causal masks are prefill-only
    assert dec(lib, mode=WINDOW_BIDIR) == UNSUPPORTED
    assert dec(lib, mode=ECP_FULL, seg=64) == UNSUPPORTED
    assert lib.sparse_attn_decode_workspace_size(2, 8, 2, 512, 128, BF16, WINDOW_BIDIR, 64, 0, 0, 0) == 0
    # s-Split decodes: split plan over the seg rows of the query's segment
    assert lib.sparse_attn_decode_workspace_size(2, 8, 2, 512, 128, BF16, SSPLIT, 0, 0, 0, 300) == \
        256 * ((2 * 8 * 3 * 132 * 4 + 255) // 256)


def opts(score_scale=0.0, cosine=0, gate_w=None, gate_b=None, out_gate=None, gate_hidden=0, gate_w2=None,
         gate_b2=None):
    return ctypes.byref(binding.SaOptions(score_scale, cosine, gate_w, gate_b, out_gate, gate_hidden, gate_w2,
                                          gate_b2))


def fwd_ex(lib, opt, q=Q, k=K, v=V, a=A, o=O, lse=None, B=1, Hq=2, Hkv=2, N=256, d=64, dtype=BF16, mode=WINDOW,
           k_win=32, pi=64, M=3, seg=0, ws=WS, wsb=1 << 30):
    return lib.sparse_attn_fwd_ex(q, k, v, a, o, lse, B, Hq, Hkv, N, d, dtype, mode, k_win, pi, M, seg, opt,
                                  ws, wsb, None)


GW, GB, OG = 0x40000000, 0x40001000, 0x50000000


@pytest.mark.parametrize("kw,okw,code", [
    (dict(), dict(score_scale=-1.0), INVALID), (dict(), dict(score_scale=float("nan")), INVALID),
    (dict(mode=PI), dict(gate_w=GW), INVALID),                 # gate_w without gate_b
    (dict(), dict(gate_w=GW, gate_b=GB), INVALID),             # the gate is a PI-mode option
    (dict(mode=PI), dict(gate_w=GW + 4, gate_b=GB), INVALID),  # misaligned (16 bytes needed)
    (dict(), dict(out_gate=OG + 8), INVALID), (dict(), dict(out_gate=O + 64), INVALID),
    (dict(ws=None, wsb=0), dict(cosine=1), WORKSPACE), (dict(ws=WS, wsb=1000), dict(cosine=1), WORKSPACE),
    (dict(ws=K + 256), dict(cosine=1), INVALID),                # the key copy would overlap k
])
def test_fwd_ex_rejects(lib, kw, okw, code):
    assert fwd_ex(lib, opts(**okw), **kw) == code


def test_fwd_ex_accepts_gate_without_alpha(lib):
    # PI with the query-driven gate needs no alpha: validation runs to the overlap check
    assert fwd_ex(lib, opts(gate_w=GW, gate_b=GB), mode=PI, a=None, o=Q) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()


def test_ex_workspace_sizes(lib):
    r256 = lambda x: -(-x // 256) * 256
    f = lib.sparse_attn_fwd_ex_workspace_size
    assert f(1, 2, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0, None) == 0
    assert f(1, 2, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0, opts(score_scale=0.3)) == 0
    assert f(1, 4, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0, opts(cosine=1)) == r256(2 * 256 * 64 * 2)
    assert f(2, 16, 16, 16384, 64, BF16, PI, 256, 1024, 15, 0, opts(cosine=1)) == \
        r256(32 * 16384 * 64 * 2) + lib.sparse_attn_fwd_workspace_size(2, 16, 16, 16384, 64, BF16, PI, 256, 1024, 15, 0)
    b = lib.sparse_attn_bwd_ex_workspace_size
    base = lib.sparse_attn_bwd_workspace_size(1, 2, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0)
    assert b(1, 2, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0, None) == base
    assert b(1, 2, 2, 256, 64, BF16, WINDOW, 32, 0, 0, 0, opts(out_gate=OG)) == base + r256(2 * 256 * 64 * 2)


def test_bwd_ex_and_decode_ex_rejects(lib):
    args = (Q, K, V, A, O, LSE, DO, DQ, DK, DV, DA, 1, 2, 2, 256, 64, BF16, PI, 32, 64, 3, 0)
    assert lib.sparse_attn_bwd_ex(*args, opts(cosine=1), None, WS, 1 << 30, None) == UNSUPPORTED
    assert lib.sparse_attn_bwd_ex(*args, opts(gate_w=GW, gate_b=GB), None, WS, 1 << 30, None) == UNSUPPORTED
    assert lib.sparse_attn_bwd_ex(*args, opts(out_gate=OG), None, WS, 1 << 30, None) == INVALID   # no dgate
    assert lib.sparse_attn_bwd_ex(*args, opts(out_gate=OG), DQ + 64, WS, 1 << 30, None) == INVALID  # dgate overlaps dq
    dargs = (Q, K, V, A, A + 4096, O, 2, 8, 2, 512, 128)
    assert lib.sparse_attn_decode_ex(*dargs, F32, PI, 64, 64, 3, 0, opts(score_scale=0.1), WS, 1 << 30, None) == UNSUPPORTED
    assert lib.sparse_attn_decode_ex(*dargs, BF16, PI, 64, 64, 3, 0, opts(out_gate=O + 16), WS, 1 << 30, None) == INVALID


def test_fwd_ex_checks_everything_before_the_first_launch(lib):
    # Cosine scores with skip keys: the workspace holds the key copy and the
    # skip state.  Too small for both must be reported before the key
    # normalisation is launched (here no device exists: a launch attempt would
    # come back as a HIP error instead of the workspace error).
    kc = 256 * (-(-(2 * 256 * 64 * 2) // 256))   # the key copy alone
    assert fwd_ex(lib, opts(cosine=1), mode=PI, ws=WS, wsb=kc) == WORKSPACE
    # the lse, alpha and out_gate regions may not overlap the workspace either
    LSE2 = WS + 4096
    assert fwd_ex(lib, opts(cosine=1), mode=PI, lse=LSE2) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()
    assert fwd_ex(lib, opts(cosine=1, out_gate=WS + 512), mode=PI) == INVALID
    assert fwd_ex(lib, opts(cosine=1), mode=PI, a=WS + 1024) == INVALID
    # an lse overlapping out_gate is rejected too
    assert fwd_ex(lib, opts(out_gate=OG), lse=OG + 64) == INVALID


def test_decode_noalloc_checks(lib):
    # the allocation-free decode: same argument checks as the decode, and
    # partial states beyond its fixed device scratch are refused before any
    # HIP call (the scratch address is looked up only after these checks)
    limit = lib.sparse_attn_decode_noalloc_max_workspace()
    assert limit == 16 << 20
    args = (Q, K, V, A + 4096, A, O)
    B = 1024
    assert lib.sparse_attn_decode_workspace_size(B, 32, 8, 32768, 128, BF16, PI, 2048, 2048, 15, 0) > limit
    assert lib.sparse_attn_decode_noalloc(*args, B, 32, 8, 32768, 128, BF16, PI, 2048, 2048, 15, 0, None) == WORKSPACE
    assert b"scratch" in lib.sparse_attn_last_error()
    assert lib.sparse_attn_decode_noalloc(*args, 2, 8, 2, 512, 96, BF16, PI, 64, 64, 3, 0, None) == UNSUPPORTED
    assert lib.sparse_attn_decode_noalloc(*args, 2, 8, 3, 512, 128, BF16, PI, 64, 64, 3, 0, None) == INVALID
    assert lib.sparse_attn_decode_noalloc(Q, K, V, A + 4096, None, O, 2, 8, 2, 512, 128, BF16, PI, 64, 64, 3, 0,
                                          None) == INVALID   # alpha required
    assert lib.sparse_attn_decode_noalloc(Q, K, V, A + 4096, A, Q, 2, 8, 2, 512, 128, BF16, PI, 64, 64, 3, 0,
                                          None) == INVALID   # o overlaps q


GW2, GB2 = 0x40002000, 0x40003000


@pytest.mark.parametrize("okw", [
    dict(gate_w=GW, gate_b=GB, gate_hidden=33, gate_w2=GW2, gate_b2=GB2),    # hidden width beyond 32
    dict(gate_w=GW, gate_b=GB, gate_hidden=-1),
    dict(gate_w=GW, gate_b=GB, gate_hidden=8, gate_b2=GB2),                  # second layer missing
    dict(gate_w=GW, gate_b=GB, gate_hidden=8, gate_w2=GW2),
    dict(gate_w=GW, gate_b=GB, gate_w2=GW2, gate_b2=GB2),                    # second layer without a width
    dict(gate_hidden=8, gate_w2=GW2, gate_b2=GB2),                           # no first layer
    dict(gate_w=GW, gate_b=GB, gate_hidden=8, gate_w2=GW2 + 2, gate_b2=GB2), # misaligned
])
def test_gate_network_option_checks(lib, okw):
    assert fwd_ex(lib, opts(**okw), mode=PI, a=None) == INVALID
    assert lib.sparse_attn_decode_ex(Q, K, V, A + 4096, None, O, 2, 8, 2, 512, 128, BF16, PI, 64, 64, 3, 0,
                                     opts(**okw), WS, 1 << 30, None) == INVALID


def test_gate_network_accepted_without_alpha(lib):
    # a complete two-layer gate needs no alpha: validation runs to the overlap check
    assert fwd_ex(lib, opts(gate_w=GW, gate_b=GB, gate_hidden=8, gate_w2=GW2, gate_b2=GB2), mode=PI, a=None,
                  o=Q) == INVALID
    assert b"overlaps" in lib.sparse_attn_last_error()
    # the backward takes no gate network
    args = (Q, K, V, A, O, LSE, DO, DQ, DK, DV, DA, 1, 2, 2, 256, 64, BF16, PI, 32, 64, 3, 0)
    assert lib.sparse_attn_bwd_ex(*args, opts(gate_w=GW, gate_b=GB, gate_hidden=8, gate_w2=GW2, gate_b2=GB2),
                                  None, WS, 1 << 30, None) == UNSUPPORTED
