"""Parity of the fused gate and epilogue options on the GPU with the fp64
oracle: score scale, scaled cosine scores, the query-driven gate (one linear
layer, or the two-layer network with a ReLU hidden layer), and the output
gate, in the forward (bf16, fp32), the decode and the backward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close, assert_grad_close
from structured_sparse_causal_amd.inputs import Workload, decode_inputs, grad_output, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def gate_params(w: Workload, seed):
    g = torch.Generator().manual_seed(seed)
    gw = (0.5 * torch.randn((w.Hq, w.d), generator=g) / np.sqrt(w.d)).float()
    gb = torch.randn((w.Hq,), generator=g).float()
    return gw, gb


def gate_mlp_params(w: Workload, H, seed):
    """Gate network weights: w1 [Hq,H,d], b1 [Hq,H], w2 [Hq,H], b2 [Hq] (fp32),
    scaled so that alpha varies over (0, 1) and both sides of the ReLUs occur."""
    g = torch.Generator().manual_seed(seed)
    w1 = (torch.randn((w.Hq, H, w.d), generator=g) / np.sqrt(w.d)).float()
    b1 = (0.5 * torch.randn((w.Hq, H), generator=g)).float()
    w2 = (1.5 * torch.randn((w.Hq, H), generator=g) / np.sqrt(H)).float()
    b2 = (0.5 * torch.randn((w.Hq,), generator=g)).float()
    return w1, b1, w2, b2


def out_gate(w: Workload, seed, shape=None):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape or (w.B, w.Hq, w.N, w.d), generator=g).to(w.torch_dtype)


CASES = [
    # (workload, options)
    (Workload("scale_window", "window", "bf16", 1, 2, 2, 700, 64, k_win=100, seed=131), dict(score_scale=0.08)),
    (Workload("cos_ecp", "ecp", "bf16", 1, 2, 2, 1000, 64, seg=96, seed=132), dict(score_scale=12.0, cosine=True)),
    (Workload("cos_pi_gqa_d128", "pi", "bf16", 1, 4, 2, 900, 128, k_win=60, pi=70, M=8, seed=133),
     dict(score_scale=10.0, cosine=True)),
    (Workload("cos_bidir_f32", "window_bidir", "f32", 1, 2, 2, 300, 64, k_win=40, seed=134),
     dict(score_scale=8.0, cosine=True)),
    (Workload("gate_pi", "pi", "bf16", 2, 2, 2, 800, 64, k_win=100, pi=128, M=5, seed=135), dict(gate=True)),
    (Workload("gate_pi_long_d128", "pi", "bf16", 1, 4, 2, 900, 128, k_win=30, pi=20, M=9, seed=136), dict(gate=True)),
    (Workload("gate_pi_f32", "pi", "f32", 1, 2, 1, 500, 64, k_win=40, pi=48, M=6, seed=137), dict(gate=True)),
    (Workload("ogate_window_d128", "window", "bf16", 1, 2, 2, 600, 128, k_win=129, seed=138), dict(ogate=True)),
    (Workload("ogate_pi_f32", "pi", "f32", 1, 2, 2, 400, 64, k_win=30, pi=64, M=4, seed=139), dict(ogate=True)),
    (Workload("all_pi", "pi", "bf16", 1, 4, 2, 1100, 64, k_win=100, pi=90, M=10, seed=140),
     dict(score_scale=9.0, cosine=True, gate=True, ogate=True)),
    # the gate network (two layers, ReLU hidden layer of width H)
    (Workload("mlp_pi", "pi", "bf16", 2, 2, 2, 800, 64, k_win=100, pi=128, M=5, seed=161), dict(mlp=16)),
    (Workload("mlp_pi_long_d128", "pi", "bf16", 1, 4, 2, 900, 128, k_win=30, pi=20, M=9, seed=162), dict(mlp=32)),
    (Workload("mlp_pi_h20_gqa", "pi", "bf16", 1, 8, 2, 1500, 64, k_win=64, pi=96, M=12, seed=163), dict(mlp=20)),
    (Workload("mlp_pi_f32", "pi", "f32", 1, 2, 1, 500, 64, k_win=40, pi=48, M=6, seed=164), dict(mlp=7)),
    (Workload("mlp_pi_f32_d128", "pi", "f32", 1, 2, 2, 300, 128, k_win=20, pi=25, M=8, seed=165), dict(mlp=13)),
    (Workload("mlp_all_pi_d128", "pi", "bf16", 1, 4, 4, 1000, 128, k_win=90, pi=100, M=7, seed=166),
     dict(score_scale=9.0, cosine=True, mlp=24, ogate=True)),
]


def gpu_and_oracle_kwargs(w, o):
    gk, ok = {}, {}
    if o.get("score_scale"):
        gk["score_scale"] = ok["scale"] = o["score_scale"]
    if o.get("cosine"):
        gk["cosine"] = ok["cosine"] = True
    if o.get("gate"):
        gw, gb = gate_params(w, w.seed + 1)
        gk["gate_w"], gk["gate_b"] = gw.to(DEV), gb.to(DEV)
        ok["gate_w"], ok["gate_b"] = gw, gb
    if o.get("mlp"):
        w1, b1, w2, b2 = gate_mlp_params(w, o["mlp"], w.seed + 3)
        gk.update(gate_w=w1.to(DEV), gate_b=b1.to(DEV), gate_w2=w2.to(DEV), gate_b2=b2.to(DEV))
        ok.update(gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2)
    if o.get("ogate"):
        g = out_gate(w, w.seed + 2)
        gk["out_gate"], ok["out_gate"] = g.to(DEV), g
    return gk, ok


@pytest.mark.parametrize("w,o", CASES, ids=[c[0].name for c in CASES])
def test_forward_options(w, o):
    say("case %s %s" % (w.name, sorted(o)))
    q, k, v, a = prefill_inputs(w)
    gk, ok = gpu_and_oracle_kwargs(w, o)
    alpha = a if w.mode == "pi" and not o.get("gate") and not o.get("mlp") else None
    out = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if alpha is None else alpha.to(DEV), **prm(w), **gk)
    torch.cuda.synchronize()
    ref = oracle.fwd(q, k, v, alpha, **prm(w), **ok)
    assert_close(out.float().cpu().numpy(), ref, w.dtype, w.name)


def test_training_forward_lse_with_cosine():
    w, o = CASES[2]
    q, k, v, a = prefill_inputs(w)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), a.to(DEV), lse=lse, score_scale=10.0, cosine=True, **prm(w))
    torch.cuda.synchronize()
    ref = oracle.lse(q, k, a, scale=10.0, cosine=True, **prm(w))
    assert np.abs(lse.cpu().numpy() - ref).max() <= 5e-3 * max(1.0, np.abs(ref).max())


DEC_CASES = [
    (Workload("dec_opt_all", "pi", "bf16", 4, 16, 4, 3000, 128, k_win=200, pi=256, M=10, decode=True, seed=141),
     dict(score_scale=11.0, cosine=True, gate=True, ogate=True)),
    (Workload("dec_opt_scale_window", "window", "bf16", 3, 8, 8, 1000, 64, k_win=300, decode=True, seed=142),
     dict(score_scale=0.05, ogate=True)),
    # the gate network: 4, 16 and 24 query heads per KV head (one, four and
    # two head chunks of a workgroup's columns)
    (Workload("dec_mlp_gqa4", "pi", "bf16", 4, 16, 4, 3000, 128, k_win=200, pi=256, M=10, decode=True, seed=171),
     dict(mlp=24)),
    (Workload("dec_mlp_gqa16_d64", "pi", "bf16", 3, 32, 2, 2000, 64, k_win=150, pi=100, M=12, decode=True,
              seed=172), dict(mlp=9)),
    (Workload("dec_mlp_gqa24_all", "pi", "bf16", 2, 48, 2, 1500, 128, k_win=100, pi=128, M=9, decode=True,
              seed=173), dict(score_scale=11.0, cosine=True, mlp=32, ogate=True)),
]


@pytest.mark.parametrize("w,o", DEC_CASES, ids=[c[0].name for c in DEC_CASES])
def test_decode_options(w, o):
    say("case %s %s" % (w.name, sorted(o)))
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens = torch.tensor([1, w.N // 3, w.N - 1, w.N][:w.B], dtype=torch.int32, device=DEV)
    gk, ok = gpu_and_oracle_kwargs(w, dict(o, ogate=False))
    if o.get("ogate"):
        g = out_gate(w, w.seed + 2, shape=(w.B, w.Hq, w.d))
        gk["out_gate"], ok["out_gate"] = g.to(DEV), g
    alpha = a if w.mode == "pi" and not o.get("gate") and not o.get("mlp") else None
    out = sa.decode(q, kc, vc, lens, alpha, **prm(w), **gk)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu(), None if alpha is None else alpha.cpu(),
                        **prm(w), **ok)
    assert_close(out.float().cpu().numpy(), ref, "bf16", w.name)


BWD_CASES = [
    (Workload("bwd_ogate_pi", "pi", "bf16", 1, 4, 2, 700, 64, k_win=100, pi=128, M=5, seed=151),
     dict(score_scale=0.2, ogate=True)),
    (Workload("bwd_ogate_window_d128", "window", "bf16", 1, 2, 2, 600, 128, k_win=200, seed=152), dict(ogate=True)),
    (Workload("bwd_scale_ecp", "ecp", "bf16", 1, 2, 2, 800, 64, seg=128, seed=153), dict(score_scale=0.06)),
]


@pytest.mark.parametrize("w,o", BWD_CASES, ids=[c[0].name for c in BWD_CASES])
def test_backward_options(w, o):
    say("case %s %s" % (w.name, sorted(o)))
    q, k, v, a = prefill_inputs(w)
    dY = grad_output(w)
    gk, ok = gpu_and_oracle_kwargs(w, o)
    alpha = a if w.mode == "pi" else None
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ad = None if alpha is None else alpha.to(DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    y = sa.fwd(qd, kd, vd, ad, lse=lse, **prm(w), **gk)
    bk = {key: gk[key] for key in ("score_scale", "out_gate") if key in gk}
    grads = sa.bwd(qd, kd, vd, ad, y, lse, dY.to(DEV), **prm(w), **bk)
    torch.cuda.synchronize()
    bok = {key: ok[key] for key in ("scale", "out_gate") if key in ok}
    ref = oracle.bwd(q, k, v, alpha, dY, **prm(w), **bok)
    names = ("dq", "dk", "dv")
    for name, got, r in zip(names, grads[:3], ref[:3]):
        assert_grad_close(got.float().cpu().numpy(), r, w.name + " " + name)
    if alpha is not None:
        assert_grad_close(grads[3].cpu().numpy(), ref[3], w.name + " dalpha")
    if o.get("ogate"):
        assert_grad_close(grads[4].float().cpu().numpy(), ref[4], w.name + " dgate")
