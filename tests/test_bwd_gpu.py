"""Parity of the HIP backward pass (and of the forward's row log-sum-exp) with
the fp64 CPU oracle, through the C ABI.

The GPU backward takes the bf16 forward output o and the fp32 lse that the
GPU forward wrote, exactly as training would; the oracle recomputes everything
in fp64 from the same input bits.  Gradients are compared with the gradient
gates of ``parity.assert_grad_close``.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close, assert_grad_close
from structured_sparse_causal_amd.inputs import WORKLOADS, Workload, grad_output, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def gpu_train_step(w: Workload, q, k, v, a, dO):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), dO.to(DEV)
    ad = None if a is None else a.to(DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    o = sa.fwd(qd, kd, vd, ad, lse=lse, **prm(w))
    grads = sa.bwd(qd, kd, vd, ad, o, lse, dod, **prm(w))
    torch.cuda.synchronize()
    return o, lse, grads


BWD_CASES = [
    Workload("bwd_pi_bf16", "pi", "bf16", 1, 2, 2, 700, 64, k_win=100, pi=128, M=5, seed=61),
    Workload("bwd_pi_gqa_d128", "pi", "bf16", 1, 4, 2, 600, 128, k_win=60, pi=70, M=8, seed=62),
    Workload("bwd_pi_overlap", "pi", "bf16", 1, 2, 1, 500, 64, k_win=100, pi=30, M=6, seed=63),
    Workload("bwd_pi_pi1", "pi", "bf16", 1, 1, 1, 300, 64, k_win=5, pi=1, M=20, seed=64),
    Workload("bwd_pi_noskip", "pi", "bf16", 2, 2, 2, 300, 64, k_win=70, pi=50, M=0, seed=65),
    Workload("bwd_pi_many_periods", "pi", "bf16", 1, 2, 1, 2100, 64, k_win=40, pi=48, M=30, seed=66),
    # residue chains longer than one 16-period tile, with GQA and d = 128
    Workload("bwd_pi_gqa_long", "pi", "bf16", 1, 4, 2, 1500, 64, k_win=20, pi=16, M=12, seed=69),
    Workload("bwd_pi_long_d128", "pi", "bf16", 1, 2, 1, 900, 128, k_win=30, pi=20, M=9, seed=70),
    Workload("bwd_window_d128", "window", "bf16", 1, 2, 2, 1000, 128, k_win=300, seed=71),
    Workload("bwd_window_gqa", "window", "bf16", 2, 4, 2, 640, 64, k_win=129, seed=72),
    Workload("bwd_window_dense", "window", "bf16", 1, 2, 2, 333, 64, k_win=5000, seed=73),
    Workload("bwd_window_tiny_n", "window", "bf16", 1, 1, 1, 1, 64, k_win=3, seed=74),
    Workload("bwd_window_k0", "window", "bf16", 1, 2, 2, 200, 64, k_win=0, seed=75),
    Workload("bwd_ecp_bf16", "ecp", "bf16", 1, 2, 2, 1000, 64, seg=96, seed=81),
    Workload("bwd_ecp_d128", "ecp", "bf16", 1, 2, 1, 700, 128, seg=200, seed=82),
    Workload("bwd_ecp_seg1", "ecp", "bf16", 1, 1, 1, 130, 64, seg=1, seed=83),
    Workload("bwd_ecp_scaled", "ecp", "bf16", 1, 2, 2, 1100, 64, seg=512, scale_inputs=True, seed=84),
]


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_bwd_parity(w):
    say("case %s" % (w,))
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    o, lse, (dq, dk, dv, da) = gpu_train_step(w, q, k, v, a, dO)
    a_or = a if w.mode == "pi" else None
    ref_o = oracle.fwd(q, k, v, a_or, **prm(w))
    assert_close(o.float().cpu().numpy(), ref_o, "bf16", w.name + " o")
    ref_lse = oracle.lse(q, k, a_or, **prm(w))
    err = np.abs(lse.cpu().numpy() - ref_lse)
    assert err.max() <= 2e-3 * max(1.0, np.abs(ref_lse).max()), (w.name, err.max())
    rq, rk, rv, ra = oracle.bwd(q, k, v, a_or, dO, **prm(w))
    assert_grad_close(dq.float().cpu().numpy(), rq, w.name + " dq")
    assert_grad_close(dk.float().cpu().numpy(), rk, w.name + " dk")
    assert_grad_close(dv.float().cpu().numpy(), rv, w.name + " dv")
    if w.mode == "pi":
        assert da is not None
        assert_grad_close(da.cpu().numpy(), ra, w.name + " dalpha")
    else:
        assert da is None


def test_bwd_window_k0_gradients():
    # With k = 0 each row attends only to itself: o = v, so dv = dO summed over
    # the query heads of a group and dq = dk = 0 up to the rounding of
    # dS = 1 * (<dO, v> - <dO, o>), whose two dot products are summed in
    # different orders (fp32).
    w = Workload("bwd_k0_gqa", "window", "bf16", 1, 4, 2, 150, 64, k_win=0, seed=76)
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    o, lse, (dq, dk, dv, da) = gpu_train_step(w, q, k, v, a, dO)
    assert torch.equal(o.cpu(), v.repeat_interleave(2, dim=1))
    assert dq.abs().max().item() < 1e-5 and dk.abs().max().item() < 1e-5
    want = dO.float().view(1, 2, 2, 150, 64).sum(2)
    assert_grad_close(dv.float().cpu().numpy(), want.numpy(), "k0 dv")


def test_bwd_alpha_one_matches_window():
    # alpha = 1 puts probability 0 on the skip keys: the gradients of q, k, v
    # are those of the window-only layer, and dalpha keeps the finite skip term.
    w = Workload("bwd_a1", "pi", "bf16", 1, 2, 2, 600, 64, k_win=50, pi=64, M=6, seed=67)
    q, k, v, _ = prefill_inputs(w)
    a = torch.ones((w.B, w.Hq, w.N), dtype=torch.float32)
    dO = grad_output(w)
    _, _, (dq, dk, dv, da) = gpu_train_step(w, q, k, v, a, dO)
    ww = w.replace(mode="window", pi=0, M=0)
    _, _, (wq, wk, wv, _) = gpu_train_step(ww, q, k, v, None, dO)
    for g, h, n in ((dq, wq, "dq"), (dk, wk, "dk"), (dv, wv, "dv")):
        assert_grad_close(g.float().cpu().numpy(), h.float().cpu().numpy(), "alpha=1 " + n)
    _, _, _, ra = oracle.bwd(q, k, v, a, dO, **prm(w))
    assert np.isfinite(ra).all() and np.abs(ra).max() > 0
    assert_grad_close(da.cpu().numpy(), ra, "alpha=1 dalpha")


def test_bwd_deterministic():
    w = BWD_CASES[1]
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    _, _, g1 = gpu_train_step(w, q, k, v, a, dO)
    _, _, g2 = gpu_train_step(w, q, k, v, a, dO)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_bwd_gqa_equals_repeated_heads():
    # A GQA layer's dk, dv are the per-group sums of the MHA gradients with the
    # KV heads repeated (the same chain rule, summed over the shared heads).
    w = Workload("bwd_gqa_rep", "pi", "bf16", 1, 4, 1, 400, 64, k_win=40, pi=50, M=4, seed=68)
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    _, _, (dq, dk, dv, da) = gpu_train_step(w, q, k, v, a, dO)
    wm = w.replace(Hkv=4)
    kr, vr = k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1)
    _, _, (mq, mk, mv, ma) = gpu_train_step(wm, q, kr, vr, a, dO)
    assert_grad_close(dq.float().cpu().numpy(), mq.float().cpu().numpy(), "gqa dq")
    assert_grad_close(da.cpu().numpy(), ma.cpu().numpy(), "gqa dalpha")
    assert_grad_close(dk.float().cpu().numpy(), mk.float().sum(1, keepdim=True).cpu().numpy(), "gqa dk")
    assert_grad_close(dv.float().cpu().numpy(), mv.float().sum(1, keepdim=True).cpu().numpy(), "gqa dv")


# ---- full-size workloads, in the launch configuration the benchmark times ----

def gpu_full_train_step(w: Workload):
    q, k, v, a = prefill_inputs(w, device=DEV)
    dO = grad_output(w, device=DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    o = sa.fwd(q, k, v, a, lse=lse, **prm(w))
    grads = sa.bwd(q, k, v, a, o, lse, dO, **prm(w))
    torch.cuda.synchronize()
    return (q, k, v, a, dO), lse, grads


@pytest.mark.parametrize("name,heads", [("ecp_bf16", [(0, 0), (3, 11)]),
                                        ("pi_bf16", [(0, 0), (1, 15)])])
def test_bwd_full_size_head_slices(name, heads):
    # Hq = Hkv for these workloads, so one (batch, head) slice is a closed
    # problem: the oracle computes its gradients exactly.
    w = WORKLOADS[name]
    say("full-size backward %s" % name)
    (q, k, v, a, dO), lse, (dq, dk, dv, da) = gpu_full_train_step(w)
    for b, h in heads:
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        a_sl = sl(a) if w.mode == "pi" else None
        ref_lse = oracle.lse(sl(q), sl(k), a_sl, **prm(w))
        assert np.abs(sl(lse).numpy() - ref_lse).max() <= 2e-3 * max(1.0, np.abs(ref_lse).max())
        rq, rk, rv, ra = oracle.bwd(sl(q), sl(k), sl(v), a_sl, sl(dO), **prm(w))
        tag = "%s b%d h%d" % (name, b, h)
        assert_grad_close(sl(dq).float().numpy(), rq, tag + " dq")
        assert_grad_close(sl(dk).float().numpy(), rk, tag + " dk")
        assert_grad_close(sl(dv).float().numpy(), rv, tag + " dv")
        if w.mode == "pi":
            assert_grad_close(sl(da).numpy(), ra, tag + " dalpha")


def test_bwd_full_size_window_subsequences():
    # Window mode is local: dq of rows [s0, s0+R) and dk, dv of keys [s0, s0+R)
    # depend only on positions [s0 - k, s0 + R + k) (every query that sees those
    # keys has its whole window there), so the oracle on that sub-sequence gives
    # their exact values.
    w = WORKLOADS["window_loop_bf16"].replace(loops=1)
    say("full-size backward %s (one layer call)" % w.name)
    (q, k, v, _, dO), _, (dq, dk, dv, _) = gpu_full_train_step(w)
    K, R = w.k_win, 384
    for h, s0 in ((0, 0), (17, 30001), (31, w.N - R)):
        lo, hi = max(0, s0 - K), min(w.N, s0 + R + K)
        sub = lambda t: t[:, h:h + 1, lo:hi].cpu()
        rq, rk, rv, _ = oracle.bwd(sub(q), sub(k), sub(v), None, sub(dO), mode="window", k_win=K)
        r0 = s0 - lo
        tag = "window h%d rows %d.." % (h, s0)
        got = lambda t: t[:, h:h + 1, s0:s0 + R].float().cpu().numpy()
        assert_grad_close(got(dq), rq[:, :, r0:r0 + R], tag + " dq")
        assert_grad_close(got(dk), rk[:, :, r0:r0 + R], tag + " dk")
        assert_grad_close(got(dv), rv[:, :, r0:r0 + R], tag + " dv")
