"""Pins for the backward pass of the fp64 oracle (CPU only).

The oracle's gradients follow the chain rule through the forward definition
(pi-Attention section 2 items 1-3 for the key set and the gate prior; ECP
section 2; LT2 section 2.1).  They are pinned here against things that do not
share its code: central finite differences of the oracle's own forward (a
different computation of the same derivative), and torch autograd through an
independent dense formulation whose mask is built from the arithmetic
distance predicate.  Plus invariants that hold exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle


def dense_bias_torch(N, mode, alpha_row, k_win=0, pi=0, M=0, seg=0):
    """[N, N] additive bias as a torch fp64 expression of alpha_row [N] (so
    autograd reaches alpha): log(alpha) on local pairs, log(1-alpha) on skip
    pairs, -inf elsewhere.  Built from the distance predicate only."""
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    dist = i - j
    neg = torch.full((N, N), -math.inf, dtype=torch.float64)
    if mode == "ecp":
        vis = (dist >= 0) & ((j // seg) >= (i // seg) - 1)
        return torch.where(vis, torch.zeros_like(neg), neg)
    local = (dist >= 0) & (dist <= k_win)
    if mode == "window":
        return torch.where(local, torch.zeros_like(neg), neg)
    skip = torch.zeros((N, N), dtype=torch.bool)
    if M > 0:
        skip = (dist > k_win) & (dist % pi == 0) & (dist // pi >= 1) & (dist // pi <= M)
    a = alpha_row[:, None].expand(N, N)
    out = torch.where(local, torch.log(a), neg)
    return torch.where(skip, torch.log1p(-a), out)


def autograd_reference(q, k, v, alpha, dO, mode, **prm):
    """Gradients of sum(dO * O) by torch autograd on dense fp64 attention."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(alpha, dtype=torch.float64, requires_grad=True) if alpha is not None else None
    kr = kt.repeat_interleave(grp, dim=1)
    vr = vt.repeat_interleave(grp, dim=1)
    outs = []
    for b in range(B):
        heads = []
        for h in range(Hq):
            arow = at[b, h] if at is not None else torch.ones(N, dtype=torch.float64)
            bias = dense_bias_torch(N, mode, arow, **prm)
            s = qt[b, h] @ kr[b, h].T / math.sqrt(d) + bias
            heads.append(torch.softmax(s, dim=-1) @ vr[b, h])
        outs.append(torch.stack(heads))
    o = torch.stack(outs)
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(),
            at.grad.numpy() if at is not None else None)


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


def rnd_alpha(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.sigmoid(torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


CASES = [
    dict(mode="pi", k_win=3, pi=5, M=3),        # skips below the window
    dict(mode="pi", k_win=4, pi=2, M=4),        # skip offsets inside the window (union)
    dict(mode="window", k_win=4),
    dict(mode="ecp", seg=4),
    dict(mode="ecp", seg=5),                    # ragged last half-segment
]


@pytest.mark.parametrize("prm", CASES, ids=lambda p: "-".join("%s%s" % kv for kv in p.items()))
@pytest.mark.parametrize("gqa", [False, True], ids=["mha", "gqa"])
def test_bwd_matches_autograd(prm, gqa):
    B, Hq, N, d = 2, 4, 23, 8
    Hkv = 2 if gqa else Hq
    q, k, v = rnd((B, Hq, N, d), 1), rnd((B, Hkv, N, d), 2), rnd((B, Hkv, N, d), 3)
    dO = rnd((B, Hq, N, d), 4)
    alpha = rnd_alpha((B, Hq, N), 5) if prm["mode"] == "pi" else None
    mode = prm["mode"]
    rest = {k_: v_ for k_, v_ in prm.items() if k_ != "mode"}
    dq, dk, dv, da = oracle.bwd(q, k, v, alpha, dO, **prm)
    rq, rk, rv, ra = autograd_reference(q, k, v, alpha, dO, mode, **rest)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert np.abs(got - ref).max() <= 1e-10 * max(1.0, np.abs(ref).max()), name
    if mode == "pi":
        assert np.abs(da - ra).max() <= 1e-10 * max(1.0, np.abs(ra).max())


def _loss(q, k, v, alpha, dO, prm):
    return float((oracle.fwd(q, k, v, alpha, **prm) * dO.astype(np.float64)).sum())


@pytest.mark.parametrize("prm", [CASES[0], CASES[1], CASES[3]], ids=["pi", "pi_overlap", "ecp"])
def test_bwd_matches_finite_differences(prm):
    """Central differences of sum(dO * O) through the oracle's forward, with
    the exact fp32 step that the perturbed input carries."""
    B, Hq, Hkv, N, d = 1, 2, 1, 12, 4
    q, k, v = rnd((B, Hq, N, d), 11), rnd((B, Hkv, N, d), 12), rnd((B, Hkv, N, d), 13)
    dO = rnd((B, Hq, N, d), 14)
    alpha = rnd_alpha((B, Hq, N), 15) if prm["mode"] == "pi" else None
    dq, dk, dv, da = oracle.bwd(q, k, v, alpha, dO, **prm)
    h = np.float32(2e-3)
    tensors = [("q", q, dq), ("k", k, dk), ("v", v, dv)]
    if alpha is not None:
        tensors.append(("alpha", alpha, da))
    for name, x, g in tensors:
        fd = np.empty_like(g)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            x0 = flat[idx]
            hp, hm = np.float32(x0 + h), np.float32(x0 - h)
            flat[idx] = hp
            lp = _loss(q, k, v, alpha, dO, prm)
            flat[idx] = hm
            lm = _loss(q, k, v, alpha, dO, prm)
            flat[idx] = x0
            fd.reshape(-1)[idx] = (lp - lm) / (float(hp) - float(hm))
        assert np.abs(fd - g).max() <= 2e-5 * max(1.0, np.abs(g).max()), name


def test_lse_matches_dense_logsumexp():
    B, Hq, Hkv, N, d = 1, 2, 1, 30, 8
    q, k = rnd((B, Hq, N, d), 21), rnd((B, Hkv, N, d), 22)
    alpha = rnd_alpha((B, Hq, N), 23)
    prm = dict(k_win=4, pi=6, M=3)
    got = oracle.lse(q, k, alpha, mode="pi", **prm)
    for h in range(Hq):
        bias = dense_bias_torch(N, "pi", torch.tensor(alpha[0, h], dtype=torch.float64), **prm)
        s = torch.tensor(q[0, h], dtype=torch.float64) @ torch.tensor(k[0, 0], dtype=torch.float64).T
        ref = torch.logsumexp(s / math.sqrt(d) + bias, dim=-1).numpy()
        assert np.abs(got[0, h] - ref).max() <= 1e-12


def test_constant_values_give_zero_score_gradients():
    """With every value row equal, O does not depend on the scores: dq, dk
    and dalpha vanish and dv_j = sum_i P_ij dO_i sums to sum_i dO_i."""
    B, Hq, N, d = 1, 2, 20, 8
    q, k = rnd((B, Hq, N, d), 31), rnd((B, Hq, N, d), 32)
    v = np.broadcast_to(rnd((1, 1, 1, d), 33), (B, Hq, N, d)).copy()
    dO = rnd((B, Hq, N, d), 34)
    alpha = rnd_alpha((B, Hq, N), 35)
    dq, dk, dv, da = oracle.bwd(q, k, v, alpha, dO, mode="pi", k_win=3, pi=4, M=4)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12 and np.abs(da).max() < 1e-12
    assert np.abs(dv.sum(axis=2) - dO.astype(np.float64).sum(axis=2)).max() < 1e-10


def test_rows_without_skips_have_zero_gate_gradient():
    B, Hq, N, d = 1, 1, 40, 8
    q, k, v, dO = (rnd((B, Hq, N, d), s) for s in (41, 42, 43, 44))
    alpha = rnd_alpha((B, Hq, N), 45)
    prm = dict(mode="pi", k_win=6, pi=10, M=2)
    _, _, _, da = oracle.bwd(q, k, v, alpha, dO, **prm)
    no_skip = [i for i in range(N) if (oracle.key_set(i, **prm)[1] == 0).all()]
    assert len(no_skip) > 5
    assert np.abs(da[0, 0, no_skip]).max() < 1e-12
    assert np.abs(da).max() > 1e-3


def test_gate_gradient_at_alpha_one_is_the_limit():
    """alpha = 1 removes the skip keys (log 0); the gate gradient there is the
    limit alpha -> 1 of the autograd gradient, and finite."""
    B, Hq, N, d = 1, 1, 25, 8
    q, k, v, dO = (rnd((B, Hq, N, d), s) for s in (51, 52, 53, 54))
    ones = np.ones((B, Hq, N), dtype=np.float32)
    prm = dict(k_win=3, pi=5, M=3)
    _, _, _, da1 = oracle.bwd(q, k, v, ones, dO, mode="pi", **prm)
    assert np.isfinite(da1).all()
    near = np.full((B, Hq, N), 1.0 - 1e-7)
    qt = torch.tensor(q, dtype=torch.float64)
    kt = torch.tensor(k, dtype=torch.float64)
    vt = torch.tensor(v, dtype=torch.float64)
    at = torch.tensor(near[0, 0], dtype=torch.float64, requires_grad=True)
    s = qt[0, 0] @ kt[0, 0].T / math.sqrt(d) + dense_bias_torch(N, "pi", at, **prm)
    o = torch.softmax(s, dim=-1) @ vt[0, 0]
    (o * torch.tensor(dO[0, 0], dtype=torch.float64)).sum().backward()
    assert np.abs(da1[0, 0] - at.grad.numpy()).max() < 1e-5
