"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Small and medium cases compare every output element; the full-size workloads,
run in the same launch configuration the benchmark times, compare sampled
rows, heads or sequences that the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import WORKLOADS, Workload, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def gpu_fwd(w: Workload, q, k, v, a, **over):
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    prm.update(over)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if a is None else a.to(DEV), **prm)
    torch.cuda.synchronize()
    return o


def oracle_fwd(w: Workload, q, k, v, a, rows=None, **over):
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    prm.update(over)
    return oracle.fwd(q, k, v, a if prm["mode"] == "pi" else None, rows=rows, **prm)


def check_full(w: Workload, **over):
    say("case %s" % (w,))
    q, k, v, a = prefill_inputs(w)
    o = gpu_fwd(w, q, k, v, a, **over)
    ref = oracle_fwd(w, q, k, v, a, **over)
    assert_close(o.float().cpu().numpy(), ref, w.dtype, w.name)
    return o, ref


CASES = [
    WORKLOADS["pi_tiny_f32"],
    Workload("pi_small_bf16", "pi", "bf16", 1, 2, 2, 1000, 64, k_win=100, pi=128, M=5, seed=21),
    Workload("pi_overlap_bf16", "pi", "bf16", 1, 2, 2, 777, 64, k_win=100, pi=30, M=6, seed=22),
    Workload("pi_pi1_bf16", "pi", "bf16", 1, 1, 1, 300, 64, k_win=5, pi=1, M=20, seed=23),
    Workload("pi_many_periods_bf16", "pi", "bf16", 1, 2, 1, 2100, 128, k_win=40, pi=48, M=30, seed=24),
    Workload("pi_nomskip_bf16", "pi", "bf16", 2, 2, 2, 500, 64, k_win=70, pi=50, M=0, seed=25),
    Workload("pi_d128_f32", "pi", "f32", 1, 2, 1, 600, 128, k_win=60, pi=100, M=4, seed=26),
    Workload("pi_f32_long", "pi", "f32", 1, 1, 1, 1500, 64, k_win=200, pi=70, M=9, seed=27),
    Workload("ecp_small_bf16", "ecp", "bf16", 1, 2, 2, 1000, 64, seg=96, seed=31),
    Workload("ecp_seg512_bf16", "ecp", "bf16", 1, 2, 2, 2100, 64, seg=512, scale_inputs=True, seed=32),
    Workload("ecp_d128_f32", "ecp", "f32", 1, 1, 1, 700, 128, seg=200, seed=33),
    Workload("ecp_seg1_bf16", "ecp", "bf16", 1, 1, 1, 130, 64, seg=1, seed=34),
    Workload("window_d128_bf16", "window", "bf16", 1, 2, 2, 3000, 128, k_win=300, seed=41),
    # d = 128 bf16 ECP: heavy-first rank order (B*H a multiple of 8, whole
    # half-segments of whole blocks) and the ragged general order
    Workload("ecp_d128_rank_bf16", "ecp", "bf16", 2, 4, 4, 1024, 128, seg=256, scale_inputs=True, seed=35),
    Workload("ecp_d128_ragged_bf16", "ecp", "bf16", 1, 3, 3, 1000, 128, seg=192, seed=36),
    Workload("window_dense_bf16", "window", "bf16", 1, 2, 2, 333, 64, k_win=5000, seed=42),
    Workload("window_gqa_bf16", "window", "bf16", 2, 4, 2, 640, 128, k_win=129, seed=43),
    Workload("window_tiny_n_bf16", "window", "bf16", 1, 1, 1, 1, 64, k_win=3, seed=44),
    Workload("window_f32", "window", "f32", 1, 2, 2, 200, 64, k_win=17, seed=45),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_parity_full(w):
    check_full(w)


def test_window_k0_is_identity_bitwise():
    w = Workload("window_k0_bf16", "window", "bf16", 1, 2, 2, 300, 64, k_win=0, seed=51)
    q, k, v, a = prefill_inputs(w)
    o = gpu_fwd(w, q, k, v, a)
    assert torch.equal(o.cpu(), v)


def test_alpha_one_equals_window_on_gpu():
    w = Workload("pi_alpha1_bf16", "pi", "bf16", 1, 2, 2, 900, 64, k_win=64, pi=100, M=6, seed=52)
    q, k, v, a = prefill_inputs(w)
    ones = torch.ones_like(a)
    o_pi = gpu_fwd(w, q, k, v, ones)
    o_win = gpu_fwd(w, q, k, v, None, mode="window")
    assert torch.equal(o_pi, o_win)


def test_tiny_alpha():
    w = Workload("pi_tiny_alpha_bf16", "pi", "bf16", 1, 2, 2, 900, 64, k_win=64, pi=100, M=6, seed=53)
    q, k, v, a = prefill_inputs(w)
    a = torch.full_like(a, 1e-3)
    o = gpu_fwd(w, q, k, v, a)
    ref = oracle_fwd(w, q, k, v, a)
    assert_close(o.float().cpu().numpy(), ref, "bf16", w.name)


def test_deterministic():
    w = Workload("pi_det_bf16", "pi", "bf16", 1, 2, 2, 1200, 64, k_win=100, pi=128, M=5, seed=54)
    q, k, v, a = prefill_inputs(w)
    o1 = gpu_fwd(w, q, k, v, a)
    o2 = gpu_fwd(w, q, k, v, a)
    assert torch.equal(o1, o2)


def test_gqa_equals_repeated_heads_on_gpu():
    w = Workload("pi_gqa_bf16", "pi", "bf16", 1, 4, 2, 500, 64, k_win=50, pi=64, M=4, seed=55)
    q, k, v, a = prefill_inputs(w)
    o = gpu_fwd(w, q, k, v, a)
    o2 = gpu_fwd(w, q, k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1), a)
    assert torch.equal(o, o2)


def test_loop_small_per_step_and_chain():
    """Looped window block (V <- O, four applications) at a reduced length."""
    w = Workload("window_loop_small", "window", "bf16", 1, 2, 2, 4096, 128, k_win=1024,
                 scale_inputs=True, loops=4, seed=56)
    q, k, v, _ = prefill_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    vin = vd
    outs = []
    for t in range(w.loops):
        o = sa.fwd(qd, kd, vin, mode="window", k_win=w.k_win)
        torch.cuda.synchronize()
        ref_t = oracle.fwd(q, k, vin.cpu(), mode="window", k_win=w.k_win)
        assert_close(o.float().cpu().numpy(), ref_t, "bf16", "loop step %d" % t)
        outs.append(o)
        vin = o
    chain = oracle.loop_fwd(q, k, v, steps=w.loops, mode="window", k_win=w.k_win)
    assert_close(outs[-1].float().cpu().numpy(), chain[-1], "bf16", "loop chain")
    last = sa.loop_fwd(qd, kd, vd, steps=w.loops, mode="window", k_win=w.k_win)
    torch.cuda.synchronize()
    assert torch.equal(last, outs[-1])


def test_loop_cone_bitwise_on_gpu():
    """After T loops of a window-k block, rows i depend only on V rows
    [i - T k, i]: perturbing earlier V rows leaves them bitwise unchanged."""
    N, kw, T = 2048, 64, 4
    w = Workload("cone", "window", "bf16", 1, 2, 2, N, 64, k_win=kw, scale_inputs=True, seed=57)
    q, k, v, _ = prefill_inputs(w)
    qd, kd = q.to(DEV), k.to(DEV)
    i0 = 1500
    v2 = v.clone()
    v2[:, :, : i0 - T * kw] = torch.randn(v2[:, :, : i0 - T * kw].shape).to(torch.bfloat16)
    o1 = sa.loop_fwd(qd, kd, v.to(DEV), steps=T, mode="window", k_win=kw).clone()
    o2 = sa.loop_fwd(qd, kd, v2.to(DEV), steps=T, mode="window", k_win=kw)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, i0:], o2[:, :, i0:])
    assert not torch.equal(o1[:, :, : i0 - T * kw], o2[:, :, : i0 - T * kw])


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
DECODE_CASES = [
    Workload("dec_pi_gqa4_bf16", "pi", "bf16", 3, 8, 2, 1000, 128, k_win=100, pi=128, M=5,
             decode=True, seed=61),
    Workload("dec_pi_overlap_bf16", "pi", "bf16", 2, 4, 4, 700, 64, k_win=96, pi=32, M=7,
             decode=True, seed=62),
    Workload("dec_window_bf16", "window", "bf16", 2, 4, 1, 3000, 128, k_win=1000, decode=True,
             seed=63),
    Workload("dec_ecp_bf16", "ecp", "bf16", 2, 6, 2, 1500, 64, seg=300, decode=True, seed=64),
    Workload("dec_pi_f32", "pi", "f32", 2, 4, 2, 500, 128, k_win=64, pi=80, M=4, decode=True,
             seed=65),
    Workload("dec_gqa32_bf16", "pi", "bf16", 1, 32, 1, 400, 64, k_win=50, pi=64, M=3,
             decode=True, seed=66),
    Workload("dec_gqa8_bf16", "pi", "bf16", 2, 16, 2, 900, 128, k_win=80, pi=100, M=6,
             decode=True, seed=69),
    Workload("dec_gqa12_bf16", "window", "bf16", 1, 12, 1, 600, 128, k_win=300, decode=True,
             seed=70),
    Workload("dec_k0_bf16", "window", "bf16", 2, 4, 2, 300, 64, k_win=0, decode=True, seed=72),
    Workload("dec_k0_pi_f32", "pi", "f32", 2, 2, 1, 300, 64, k_win=0, pi=37, M=5, decode=True,
             seed=73),
]


def gpu_decode(w, q, kc, vc, lens, a):
    o = sa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV),
                  None if a is None else a.to(DEV), mode=w.mode, k_win=w.k_win, pi=w.pi,
                  M=w.M, seg=w.seg)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("w", DECODE_CASES, ids=lambda w: w.name)
def test_decode_parity(w):
    say("case %s" % (w,))
    q, kc, vc, lens, a = decode_inputs(w)
    # ragged lengths: full, short, a single token and one just past a skip boundary
    choices = [w.N, max(1, w.N // 3), 1, min(w.N, w.pi * 2 + w.k_win + 2) if w.pi else w.N]
    lens = torch.tensor([choices[b % len(choices)] for b in range(w.B)], dtype=torch.int32)
    o = gpu_decode(w, q, kc, vc, lens, a)
    ref = oracle.decode(q, kc, vc, lens, a if w.mode == "pi" else None, mode=w.mode,
                        k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    assert_close(o.float().cpu().numpy(), ref, w.dtype, w.name)


def test_decode_equals_prefill_row():
    w = Workload("dec_vs_prefill", "pi", "bf16", 1, 4, 4, 1500, 64, k_win=100, pi=128, M=5,
                 seed=67)
    q, k, v, a = prefill_inputs(w)
    o = gpu_fwd(w, q, k, v, a)
    L = 1234
    lens = torch.tensor([L], dtype=torch.int32)
    od = sa.decode(q[:, :, L - 1].contiguous().to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV),
                   a[:, :, L - 1].contiguous().to(DEV), mode="pi", k_win=w.k_win, pi=w.pi, M=w.M)
    torch.cuda.synchronize()
    diff = (od.float() - o[:, :, L - 1].float()).abs().max().item()
    assert diff <= 1e-2, diff


def test_decode_bad_length_gives_nan_not_fault():
    w = Workload("dec_badlen", "window", "bf16", 2, 2, 2, 256, 64, k_win=16, decode=True, seed=68)
    q, kc, vc, lens, a = decode_inputs(w)
    lens = torch.tensor([0, 300], dtype=torch.int32)
    o = gpu_decode(w, q, kc, vc, lens, None)
    assert torch.isnan(o.float()).all()


# ---------------------------------------------------------------------------
# Full-size workloads, sampled (same launch configuration as the benchmark)
# ---------------------------------------------------------------------------
def _sample_rows(rng, B, H, N, n, hs=None):
    b = rng.integers(0, B, n)
    h = rng.integers(0, H, n) if hs is None else rng.choice(hs, n)
    i = np.concatenate([rng.integers(0, N, n - 6), [0, 1, N - 1, N - 2, N // 2, 127]])
    return (b * H + h) * N + i


@pytest.mark.parametrize("name", ["ecp_bf16", "pi_bf16"])
def test_full_size_every_row(name):
    # every output element of the full workload (about 35 GFLOP of fp64 work
    # for the oracle, seconds on the host's cores)
    w = WORKLOADS[name]
    say("full-size %s, every row" % name)
    q, k, v, a = prefill_inputs(w, device=DEV)
    o = gpu_fwd(w, q, k, v, a).float().cpu().numpy()
    ref = oracle_fwd(w, q.cpu(), k.cpu(), v.cpu(), None if a is None else a.cpu())
    assert_close(o, ref, "bf16", name)


def test_pi_gqa_several_chunks_sampled():
    """pi-Attention with GQA large enough that the skip pass and the prefill run
    over several chunks of head groups (workspace reused between chunks)."""
    w = Workload("pi_gqa_chunks", "pi", "bf16", 2, 32, 8, 32768, 64, k_win=200, pi=700, M=20,
                 seed=71)
    say("chunked %s" % (w,))
    whole = w.B * w.Hq * w.N * (8 + 2 * w.d)          # skip state of every row at once
    assert 0 < sa.fwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, torch.bfloat16, "pi", w.k_win,
                                    w.pi, w.M) < whole / 2
    q, k, v, a = prefill_inputs(w, device=DEV)
    o = gpu_fwd(w, q, k, v, a).float().cpu().numpy().reshape(-1, w.d)
    rows = _sample_rows(np.random.default_rng(7), w.B, w.Hq, w.N, 3000)
    ref = oracle_fwd(w, q.cpu(), k.cpu(), v.cpu(), a.cpu(), rows=rows)
    assert_close(o[rows], ref, "bf16", w.name)


def test_full_size_window_loop_sampled():
    w = WORKLOADS["window_loop_bf16"]
    say("full-size %s" % w.name)
    qd, kd, vd, _ = prefill_inputs(w, device=DEV)
    q, k = qd.cpu(), kd.cpu()
    vin = vd
    rng = np.random.default_rng(6)
    heads = [0, 5, 9, 14, 17, 22, 27, 31]
    for t in range(w.loops):
        o = sa.fwd(qd, kd, vin, mode="window", k_win=w.k_win)
        torch.cuda.synchronize()
        for h in heads:
            rows = np.concatenate([rng.integers(0, w.N, 1500), [0, 1, w.N - 1, 1024, 1025],
                                   np.arange(1000, 1160)])
            ref = oracle.fwd(q[:, h:h + 1], k[:, h:h + 1], vin[:, h:h + 1].cpu(), mode="window",
                             k_win=w.k_win, rows=rows)
            got = o[0, h, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
            assert_close(got, ref, "bf16", "loop step %d head %d" % (t, h))
        vin = o


def test_full_size_decode_every_sequence():
    # all 64 sequences, with the benchmark's full caches and then with ragged
    # lengths (including 1, the window edge and the skip edge); the oracle
    # reads each sequence's cache slice from the host
    w = WORKLOADS["decode_pi_gqa_bf16"]
    say("full-size %s, every sequence" % w.name)
    q, kc, vc, lens, a = decode_inputs(w, device=DEV)
    rng = np.random.default_rng(11)
    ragged = rng.integers(1, w.N + 1, w.B)
    ragged[:6] = [1, 2, w.k_win, w.k_win + 2, w.pi * 3 + 1, w.N]
    prm = dict(mode="pi", k_win=w.k_win, pi=w.pi, M=w.M)
    for tag, ln in (("full", lens), ("ragged", torch.from_numpy(ragged.astype(np.int32)).to(DEV))):
        o = sa.decode(q, kc, vc, ln, a, **prm).float().cpu().numpy()
        lnc = ln.cpu()
        for b0 in range(0, w.B, 8):
            say("  %s sequences %d..%d" % (tag, b0, b0 + 7))
            sl = slice(b0, b0 + 8)
            ref = oracle.decode(q[sl].cpu(), kc[sl].cpu(), vc[sl].cpu(), lnc[sl], a[sl].cpu(), **prm)
            assert_close(o[sl], ref, "bf16", "decode %s seq %d..%d" % (tag, b0, b0 + 7))
