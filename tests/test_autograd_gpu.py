"""The differentiable entry ``attention`` (torch autograd over the training
forward and the backward) against the fp64 oracle, the looped block trained
through its applications, and the two compositions it is meant for: scaled
cosine scores formed by normalising q and k in the caller, and a gate network
on the query formed in the caller.  In both the
caller's own autograd carries the library's gradients (of the normalised
rows, of alpha) back to its parameters; the references apply the same
chain rule in fp64 to the oracle's gradients."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_grad_close
from structured_sparse_causal_amd.inputs import Workload, grad_output, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def leaf(t, dtype=None):
    return t.to(DEV, dtype=dtype or t.dtype).detach().requires_grad_(True)


@pytest.mark.parametrize("w", [
    Workload("ag_pi_gqa", "pi", "bf16", 1, 4, 2, 700, 64, k_win=100, pi=128, M=5, seed=181),
    Workload("ag_ecp_d128", "ecp", "bf16", 2, 2, 2, 600, 128, seg=80, seed=182),
    Workload("ag_window", "window", "bf16", 1, 2, 1, 500, 64, k_win=64, seed=183),
], ids=lambda w: w.name)
def test_attention_autograd(w):
    print("case %s" % (w,), flush=True)
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)                                   # bf16, the gradient the loss sends to o
    qd, kd, vd = leaf(q), leaf(k), leaf(v)
    ad = leaf(a) if a is not None else None
    o = sa.attention(qd, kd, vd, ad, **prm(w))
    # sum(o * dO) has gradient dO (exact: dO is bf16 and o is bf16)
    (o.float() * dO.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    # the same gradients as the direct entry points (same kernels, same inputs)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    ad0 = a.to(DEV) if a is not None else None
    o2 = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), ad0, lse=lse, **prm(w))
    g2 = sa.bwd(q.to(DEV), k.to(DEV), v.to(DEV), ad0, o2, lse, dO.to(DEV), **prm(w))
    assert torch.equal(o.detach(), o2)
    assert torch.equal(qd.grad, g2[0]) and torch.equal(kd.grad, g2[1]) and torch.equal(vd.grad, g2[2])
    if a is not None:
        assert torch.equal(ad.grad, g2[3])
    # and against the oracle's fp64 chain rule
    a_or = a if w.mode == "pi" else None
    rq, rk, rv, ra = oracle.bwd(q, k, v, a_or, dO, **prm(w))
    assert_grad_close(qd.grad.float().cpu().numpy(), rq, w.name + " dq")
    assert_grad_close(kd.grad.float().cpu().numpy(), rk, w.name + " dk")
    assert_grad_close(vd.grad.float().cpu().numpy(), rv, w.name + " dv")
    if a is not None:
        assert_grad_close(ad.grad.cpu().numpy(), ra, w.name + " dalpha")


def test_attention_autograd_output_gate():
    w = Workload("ag_ogate_pi", "pi", "bf16", 1, 2, 2, 600, 64, k_win=90, pi=100, M=5, seed=184)
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    g = torch.Generator().manual_seed(185)
    gate = torch.randn((w.B, w.Hq, w.N, w.d), generator=g).bfloat16()
    qd, kd, vd, ad, gd = leaf(q), leaf(k), leaf(v), leaf(a), leaf(gate)
    y = sa.attention(qd, kd, vd, ad, out_gate=gd, **prm(w))
    (y.float() * dO.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    rq, rk, rv, ra, rg = oracle.bwd(q, k, v, a, dO, out_gate=gate, **prm(w))
    assert_grad_close(qd.grad.float().cpu().numpy(), rq, "ogate dq")
    assert_grad_close(kd.grad.float().cpu().numpy(), rk, "ogate dk")
    assert_grad_close(vd.grad.float().cpu().numpy(), rv, "ogate dv")
    assert_grad_close(ad.grad.cpu().numpy(), ra, "ogate dalpha")
    assert_grad_close(gd.grad.float().cpu().numpy(), rg, "ogate dgate")


def _normalise_backward(x, gx):
    """Chain rule of x -> x / |x| (last axis), fp64: gx is the gradient of the
    normalised rows, the result the gradient of x."""
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    xh = x / n
    return (gx - xh * np.sum(xh * gx, axis=-1, keepdims=True)) / n


def test_cosine_scores_by_composition():
    # tau * cos(q_i, k_j): the caller normalises q and k (fp32, rounded to
    # bf16 for the library) and passes tau as the score scale.
    w = Workload("ag_cos_ecp", "ecp", "bf16", 1, 2, 2, 700, 64, seg=96, seed=186)
    tau = 10.0
    q, k, v, _ = prefill_inputs(w)
    dO = grad_output(w)
    qr, kr = leaf(q, torch.float32), leaf(k, torch.float32)
    vd = leaf(v)
    qn = torch.nn.functional.normalize(qr, dim=-1).bfloat16()
    kn = torch.nn.functional.normalize(kr, dim=-1).bfloat16()
    o = sa.attention(qn, kn, vd, mode=w.mode, seg=w.seg, score_scale=tau)
    (o.float() * dO.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    qn_c, kn_c = qn.detach().cpu(), kn.detach().cpu()
    rqn, rkn, rv, _ = oracle.bwd(qn_c, kn_c, v, None, dO, mode=w.mode, seg=w.seg, scale=tau)
    q64, k64 = q.double().numpy(), k.double().numpy()
    assert_grad_close(qr.grad.cpu().numpy(), _normalise_backward(q64, rqn), "cosine dq")
    assert_grad_close(kr.grad.cpu().numpy(), _normalise_backward(k64, rkn), "cosine dk")
    assert_grad_close(vd.grad.float().cpu().numpy(), rv, "cosine dv")


def test_gate_network_by_composition():
    # alpha = sigmoid(w2 . relu(W1 q + b1) + b2) per head, formed by the caller
    # (fp32 on the GPU); its parameters get their gradients from dalpha.
    w = Workload("ag_mlp_pi", "pi", "bf16", 1, 2, 2, 800, 64, k_win=100, pi=128, M=5, seed=187)
    H = 16
    q, k, v, _ = prefill_inputs(w)
    dO = grad_output(w)
    g = torch.Generator().manual_seed(188)
    w1 = (torch.randn((w.Hq, H, w.d), generator=g) / np.sqrt(w.d)).float()
    b1 = (0.5 * torch.randn((w.Hq, H), generator=g)).float()
    w2 = (1.5 * torch.randn((w.Hq, H), generator=g) / np.sqrt(H)).float()
    b2 = (0.5 * torch.randn((w.Hq,), generator=g)).float()

    def gate(qf, w1, b1, w2, b2):
        # (fp32 / fp64 products only; the weights' transpose made contiguous)
        hid = torch.relu(torch.matmul(qf, w1.transpose(-1, -2).contiguous()[None]) + b1[None, :, None, :])
        return torch.sigmoid((hid * w2[None, :, None, :]).sum(-1) + b2[None, :, None])

    params = [leaf(t) for t in (w1, b1, w2, b2)]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    alpha = gate(qd.float(), *params).contiguous()
    o = sa.attention(qd, kd, vd, alpha, **prm(w))
    (o.float() * dO.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    # reference: the oracle's dalpha at the same alpha, carried through the
    # gate network in fp64 on the host
    a_used = alpha.detach().cpu()
    _, _, _, ra = oracle.bwd(q, k, v, a_used, dO, **prm(w))
    p64 = [t.double().requires_grad_(True) for t in (w1, b1, w2, b2)]
    a64 = gate(q.double(), *p64)
    ref = torch.autograd.grad(a64, p64, grad_outputs=torch.from_numpy(np.asarray(ra, dtype=np.float64)))
    for name, got, r in zip(("w1", "b1", "w2", "b2"), params, ref):
        assert_grad_close(got.grad.cpu().numpy(), r.numpy(), "gate network d" + name)


def test_looped_block_autograd():
    # The looped block (LT2 section 2.2): V_{t+1} = O_t (bf16, as stored) with q
    # and k fixed, trained through all T applications.  Reference: the oracle's
    # forward chain (rounded to bf16 between applications, as the looped
    # oracle does) and its backward applied in reverse, dq and dk summed over
    # the applications and each application's dv fed to the one before.
    w = Workload("ag_loop", "window", "bf16", 1, 2, 2, 600, 64, k_win=64, seed=189)
    T = 3
    q, k, v, _ = prefill_inputs(w)
    dO = grad_output(w)
    qd, kd, vd = leaf(q), leaf(k), leaf(v)
    x = vd
    for _ in range(T):
        x = sa.attention(qd, kd, x, mode="window", k_win=w.k_win)
    (x.float() * dO.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    vs = [v]
    for _ in range(T - 1):
        vs.append(torch.from_numpy(oracle.fwd(q, k, vs[-1], mode="window", k_win=w.k_win)).float().bfloat16())
    g = dO.float()
    rq = rk = 0.0
    for t in reversed(range(T)):
        gq, gk, gv, _ = oracle.bwd(q, k, vs[t], None, g, mode="window", k_win=w.k_win)
        rq, rk, g = rq + gq, rk + gk, torch.from_numpy(np.asarray(gv)).float()
    assert_grad_close(qd.grad.float().cpu().numpy(), rq, "loop dq")
    assert_grad_close(kd.grad.float().cpu().numpy(), rk, "loop dk")
    assert_grad_close(vd.grad.float().cpu().numpy(), g.numpy(), "loop dv")
