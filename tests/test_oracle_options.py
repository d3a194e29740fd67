"""Pins for the oracle's fused gate and epilogue options (CPU only).

    scale      score scale other than 1/sqrt(d)
    cosine     scores scale * cos(q_i, k_j) (scaled cosine attention, the
               attention branch of the hybrid GSS-Transformer page)
    gate_w/b   alpha = sigmoid(<w_h, q_i> + b_h) from the query (pi-Attention
               section 2 item 3: a light network per token and head)
    gate MLP   alpha = sigmoid(sum_u w2_hu relu(<w1_hu, q_i> + b1_hu) + b2_h):
               the same network with a ReLU hidden layer
    out_gate   y = o * sigmoid(g) (LT2 page, section 3: SDPA output gate)

Pinned against torch's scaled_dot_product_attention (its ``scale`` argument,
F.normalize'd inputs), invariances, the explicit-alpha path, and torch
autograd for the gradients.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


def t64(x):
    return torch.tensor(x, dtype=torch.float64)


def test_scale_matches_sdpa():
    q, k, v = rnd((1, 2, 21, 8), 1), rnd((1, 2, 21, 8), 2), rnd((1, 2, 21, 8), 3)
    for sc in (0.05, 0.7):
        ref = F.scaled_dot_product_attention(t64(q), t64(k), t64(v), is_causal=True, scale=sc).numpy()
        got = oracle.fwd(q, k, v, mode="window", k_win=100, scale=sc)
        assert np.abs(got - ref).max() < 1e-12


def test_cosine_matches_sdpa_on_normalised_inputs():
    q, k, v = rnd((1, 2, 25, 16), 4), rnd((1, 2, 25, 16), 5), rnd((1, 2, 25, 16), 6)
    tau = 7.5
    ref = F.scaled_dot_product_attention(F.normalize(t64(q), dim=-1), F.normalize(t64(k), dim=-1), t64(v),
                                         is_causal=True, scale=tau).numpy()
    got = oracle.fwd(q, k, v, mode="window", k_win=100, scale=tau, cosine=True)
    assert np.abs(got - ref).max() < 1e-12


def test_cosine_is_invariant_to_row_scaling():
    q, k, v = rnd((1, 2, 30, 8), 7), rnd((1, 2, 30, 8), 8), rnd((1, 2, 30, 8), 9)
    a = np.abs(rnd((1, 2, 30, 1), 10)) + 0.25
    c = np.abs(rnd((1, 2, 30, 1), 11)) + 0.25
    prm = dict(mode="pi", k_win=4, pi=6, M=3, scale=3.0, cosine=True)
    alpha = 1.0 / (1.0 + np.exp(-rnd((1, 2, 30), 12)))
    o1 = oracle.fwd(q, k, v, alpha, **prm)
    o2 = oracle.fwd((q * a).astype(np.float32), (k * c).astype(np.float32), v, alpha, **prm)
    assert np.abs(o1 - o2).max() < 1e-6          # rows rescaled in fp32: rounding only


def test_query_gate_equals_explicit_alpha():
    B, H, N, d = 1, 3, 40, 16
    q, k, v = rnd((B, H, N, d), 13), rnd((B, H, N, d), 14), rnd((B, H, N, d), 15)
    w, b = rnd((H, d), 16, 0.3), rnd((H,), 17)
    prm = dict(mode="pi", k_win=5, pi=7, M=4)
    got = oracle.fwd(q, k, v, None, gate_w=w, gate_b=b, **prm)
    alpha = torch.sigmoid(torch.einsum("bhnd,hd->bhn", t64(q), t64(w)) + t64(b)[None, :, None]).numpy()
    ref = oracle.fwd(q, k, v, alpha.astype(np.float32), **prm)
    assert np.abs(got - ref).max() < 1e-6        # alpha passed as fp32 on the explicit path
    # zero weights: alpha = sigmoid(b_h), the same for every token of a head
    const = oracle.fwd(q, k, v, None, gate_w=np.zeros((H, d), np.float32), gate_b=b, **prm)
    ab = np.broadcast_to(1.0 / (1.0 + np.exp(-b.astype(np.float64)))[None, :, None], (B, H, N))
    assert np.abs(const - oracle.fwd(q, k, v, ab.astype(np.float32), **prm)).max() < 1e-6
    # decode sees the same gate
    lens = np.array([N], dtype=np.int32)
    dec = oracle.decode(np.ascontiguousarray(q[:, :, -1]), k, v, lens, gate_w=w, gate_b=b, **prm)
    assert np.abs(dec - got[:, :, -1]).max() < 1e-12


def test_out_gate_forward_and_gradients_match_autograd():
    B, Hq, Hkv, N, d = 1, 4, 2, 19, 8
    q, k, v = rnd((B, Hq, N, d), 18), rnd((B, Hkv, N, d), 19), rnd((B, Hkv, N, d), 20)
    g, dY = rnd((B, Hq, N, d), 21), rnd((B, Hq, N, d), 22)
    k_win, sc = 5, 0.4
    y = oracle.fwd(q, k, v, mode="window", k_win=k_win, scale=sc, out_gate=g)
    dq, dk, dv, _, dg = oracle.bwd(q, k, v, None, dY, mode="window", k_win=k_win, scale=sc, out_gate=g)
    qt, kt, vt, gt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g))
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    mask = (i - j >= 0) & (i - j <= k_win)
    s = qt @ kt.repeat_interleave(2, 1).transpose(-1, -2) * sc
    o = torch.softmax(s.masked_fill(~mask, -math.inf), -1) @ vt.repeat_interleave(2, 1)
    yt = o * torch.sigmoid(gt)
    assert np.abs(y - yt.detach().numpy()).max() < 1e-12
    (yt * t64(dY)).sum().backward()
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad), (dg, gt.grad)):
        assert np.abs(got - ref.numpy()).max() < 1e-10 * max(1.0, ref.abs().max().item())


def test_decode_options_equal_last_prefill_row():
    N, d = 33, 16
    q, k, v = rnd((2, 4, N, d), 23), rnd((2, 2, N, d), 24), rnd((2, 2, N, d), 25)
    g = rnd((2, 4, N, d), 26)
    prm = dict(mode="window", k_win=9, scale=5.0, cosine=True)
    full = oracle.fwd(q, k, v, out_gate=g, **prm)
    lens = np.array([N, N], dtype=np.int32)
    dec = oracle.decode(np.ascontiguousarray(q[:, :, -1]), k, v, lens,
                        out_gate=np.ascontiguousarray(g[:, :, -1]), **prm)
    assert np.abs(dec - full[:, :, -1]).max() < 1e-12


def gate_mlp_alpha(q, w1, b1, w2, b2):
    """alpha of the gate MLP in fp64 by torch: [B,Hq,N] from q [B,Hq,N,d],
    w1 [Hq,H,d], b1 [Hq,H], w2 [Hq,H], b2 [Hq]."""
    hid = torch.relu(torch.einsum("bhnd,hud->bhnu", t64(q), t64(w1)) + t64(b1)[None, :, None, :])
    return torch.sigmoid((hid * t64(w2)[None, :, None, :]).sum(-1) + t64(b2)[None, :, None]).numpy()


def test_gate_mlp_equals_explicit_alpha():
    # alpha computed independently (torch, fp64) and passed on the pinned
    # explicit-alpha path: the gate network enters only through alpha
    B, H, N, d, Hg = 2, 3, 45, 16, 7
    q, k, v = rnd((B, H, N, d), 31), rnd((B, H, N, d), 32), rnd((B, H, N, d), 33)
    w1, b1 = rnd((H, Hg, d), 34, 0.4), rnd((H, Hg), 35, 0.5)
    w2, b2 = rnd((H, Hg), 36, 0.4), rnd((H,), 37, 0.3)
    prm = dict(mode="pi", k_win=4, pi=6, M=5)
    alpha = gate_mlp_alpha(q, w1, b1, w2, b2)
    assert 0.01 < alpha.min() and alpha.max() < 0.99 and alpha.std() > 0.1   # varied, not saturated
    relu_off = (np.einsum("bhnd,hud->bhnu", q.astype(np.float64), w1) + b1[None, :, None, :]) <= 0
    assert 0.2 < relu_off.mean() < 0.8                          # both sides of every ReLU are used
    got = oracle.fwd(q, k, v, None, gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2, **prm)
    ref = oracle.fwd(q, k, v, alpha.astype(np.float32), **prm)
    assert np.abs(got - ref).max() < 1e-6                       # alpha passed as fp32 on the explicit path
    lse = oracle.lse(q, k, None, gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2, **prm)
    assert np.abs(lse - oracle.lse(q, k, alpha.astype(np.float32), **prm)).max() < 1e-6
    lens = np.array([N, 17], dtype=np.int32)
    qd = np.ascontiguousarray(np.stack([q[0, :, N - 1], q[1, :, 16]]))
    dec = oracle.decode(qd, k, v, lens, gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2, **prm)
    assert np.abs(dec[0] - got[0, :, N - 1]).max() < 1e-12
    assert np.abs(dec[1] - oracle.fwd(q[:, :, :17].copy(), k[:, :, :17].copy(), v[:, :, :17].copy(), None,
                                      gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2, **prm)[1, :, 16]).max() < 1e-12


def test_gate_mlp_reduces_to_the_linear_gate():
    # relu(z) - relu(-z) = z: hidden rows (w, -w), biases (b, -b) and output
    # weights (1, -1) give the one-layer gate sigmoid(<w, q> + b) exactly
    B, H, N, d = 1, 2, 30, 8
    q, k, v = rnd((B, H, N, d), 41), rnd((B, H, N, d), 42), rnd((B, H, N, d), 43)
    w, b = rnd((H, d), 44, 0.3), rnd((H,), 45)
    w1 = np.ascontiguousarray(np.stack([w, -w], axis=1))
    b1 = np.ascontiguousarray(np.stack([b, -b], axis=1))
    w2 = np.tile(np.array([1.0, -1.0], np.float32), (H, 1))
    b2 = np.zeros(H, np.float32)
    prm = dict(mode="pi", k_win=3, pi=5, M=4)
    lin = oracle.fwd(q, k, v, None, gate_w=w, gate_b=b, **prm)
    mlp = oracle.fwd(q, k, v, None, gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2, **prm)
    assert np.abs(lin - mlp).max() < 1e-14


def test_gate_mlp_worked_example_e1():
    # Q = K = 0: the network sees only its biases.  With hidden biases (1, 2),
    # output weights (0.5, -0.3) and b2 = ln(1/3) + 0.1 the logit is ln(1/3),
    # alpha = 1/4, and the output is worked example E1 (tests/golden).
    import pathlib
    fx = {}
    for line in (pathlib.Path(__file__).parent / "golden" / "e1_pi_no_overlap.txt").read_text().splitlines():
        if line and not line.startswith("#"):
            key, *vals = line.split()
            fx[key] = vals
    N, d, H = int(fx["N"][0]), 4, 1
    q = np.zeros((1, H, N, d), np.float32)
    v = np.repeat(np.arange(N, dtype=np.float32)[None, None, :, None], d, axis=3)
    w1 = rnd((H, 2, d), 51)                                     # multiplies q = 0: any weights
    b1 = np.array([[1.0, 2.0]], np.float32)
    w2 = np.array([[0.5, -0.3]], np.float32)
    b2 = np.array([math.log(1.0 / 3.0) + 0.1], np.float32)
    o = oracle.fwd(q, q, v, None, mode="pi", k_win=int(fx["k_win"][0]), pi=int(fx["pi"][0]), M=int(fx["M"][0]),
                   gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2)
    expected = np.array([float(x) for x in fx["expected"]])
    assert np.abs(o[0, 0, :, 0] - expected).max() < 1e-6      # b2 rounded to fp32: alpha = 1/4 to ~1e-8


def test_gate_mlp_argument_checks():
    q = rnd((1, 2, 8, 4), 61)
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, None, mode="pi", k_win=1, pi=3, M=2, gate_w=rnd((2, 3, 4), 62),
                   gate_b=rnd((2, 3), 63), gate_w2=rnd((2, 2), 64), gate_b2=rnd((2,), 65))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, None, mode="pi", k_win=1, pi=3, M=2, gate_w=rnd((2, 4), 62),
                   gate_b=rnd((2,), 63), gate_b2=rnd((2,), 65))
