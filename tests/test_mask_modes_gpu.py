"""Parity of the further mask modes on the GPU (two-sided window, s-Split
segments, ECP pair without the causal mask) with the fp64 oracle: forward
(bf16 and fp32), backward (bf16), and s-Split decode."""
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
    return dict(mode=w.mode, k_win=w.k_win, seg=w.seg)


FWD_CASES = [
    Workload("bidir_bf16", "window_bidir", "bf16", 1, 2, 2, 1000, 64, k_win=100, seed=101),
    Workload("bidir_gqa_d128", "window_bidir", "bf16", 2, 4, 2, 777, 128, k_win=300, seed=102),
    Workload("bidir_dense", "window_bidir", "bf16", 1, 2, 1, 333, 64, k_win=5000, seed=103),
    Workload("bidir_f32", "window_bidir", "f32", 1, 2, 2, 300, 64, k_win=40, seed=104),
    Workload("ssplit_bf16", "ssplit", "bf16", 1, 2, 2, 1000, 64, seg=96, seed=105),
    Workload("ssplit_d128_gqa", "ssplit", "bf16", 1, 4, 1, 700, 128, seg=200, seed=106),
    Workload("ssplit_f32", "ssplit", "f32", 1, 2, 2, 260, 128, seg=50, seed=107),
    Workload("ecpfull_bf16", "ecp_full", "bf16", 1, 2, 2, 1000, 64, seg=96, seed=108),
    Workload("ecpfull_seg512", "ecp_full", "bf16", 1, 2, 2, 2100, 64, seg=512, scale_inputs=True, seed=109),
    Workload("ecpfull_gqa_d128", "ecp_full", "bf16", 2, 4, 2, 640, 128, seg=128, seed=110),
    Workload("ecpfull_f32", "ecp_full", "f32", 1, 1, 1, 300, 128, seg=64, seed=111),
]


@pytest.mark.parametrize("w", FWD_CASES, ids=lambda w: w.name)
def test_forward_parity(w):
    say("case %s" % (w,))
    q, k, v, _ = prefill_inputs(w)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), **prm(w))
    torch.cuda.synchronize()
    assert_close(o.float().cpu().numpy(), oracle.fwd(q, k, v, **prm(w)), w.dtype, w.name)


def test_identity_masks_bitwise():
    # k = 0 (two-sided) and s = 1 (s-Split) leave each query with only itself
    w = Workload("ident", "window_bidir", "bf16", 1, 2, 2, 300, 64, k_win=0, seed=112)
    q, k, v, _ = prefill_inputs(w)
    for p in (dict(mode="window_bidir", k_win=0), dict(mode="ssplit", seg=1)):
        o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), **p)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), v)


def test_bidir_reversal_symmetry_on_gpu():
    w = FWD_CASES[0]
    q, k, v, _ = prefill_inputs(w)
    flip = lambda x: x.flip(2).contiguous().to(DEV)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), **prm(w)).float().cpu()
    o_r = sa.fwd(flip(q), flip(k), flip(v), **prm(w)).float().cpu().flip(2)
    assert (o - o_r).abs().max().item() < 2e-2


BWD_CASES = [
    Workload("bwd_bidir_gqa", "window_bidir", "bf16", 1, 4, 2, 700, 64, k_win=100, seed=121),
    Workload("bwd_bidir_d128", "window_bidir", "bf16", 1, 2, 2, 500, 128, k_win=170, seed=122),
    Workload("bwd_ssplit_d128", "ssplit", "bf16", 1, 2, 2, 1000, 128, seg=96, seed=123),
    Workload("bwd_ssplit_gqa", "ssplit", "bf16", 2, 4, 1, 600, 64, seg=200, seed=124),
    Workload("bwd_ecpfull_gqa", "ecp_full", "bf16", 1, 4, 2, 1000, 64, seg=96, seed=125),
    Workload("bwd_ecpfull_seg1", "ecp_full", "bf16", 1, 1, 1, 130, 64, seg=1, seed=126),
    Workload("bwd_ecpfull_d128", "ecp_full", "bf16", 1, 2, 2, 900, 128, seg=256, seed=127),
]


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_backward_parity(w):
    say("case %s" % (w,))
    q, k, v, _ = prefill_inputs(w)
    dO = grad_output(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    o = sa.fwd(qd, kd, vd, lse=lse, **prm(w))
    dq, dk, dv, da = sa.bwd(qd, kd, vd, None, o, lse, dO.to(DEV), **prm(w))
    torch.cuda.synchronize()
    assert da is None
    ref_lse = oracle.lse(q, k, None, **prm(w))
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 2e-3 * max(1.0, np.abs(ref_lse).max())
    rq, rk, rv, _ = oracle.bwd(q, k, v, None, dO, **prm(w))
    assert_grad_close(dq.float().cpu().numpy(), rq, w.name + " dq")
    assert_grad_close(dk.float().cpu().numpy(), rk, w.name + " dk")
    assert_grad_close(dv.float().cpu().numpy(), rv, w.name + " dv")


def test_ssplit_decode():
    # s-Split is causal, so it decodes: contiguous cache and ring of seg rows
    w = Workload("dec_ssplit", "ssplit", "bf16", 4, 8, 2, 1500, 128, seg=300, decode=True, seed=128)
    q, kc, vc, _, _ = decode_inputs(w, device=DEV)
    lens = [1, 300, 301, 1500]
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = sa.decode(q, kc, vc, lens_t, mode="ssplit", seg=w.seg)
    R = w.seg
    rings = []
    for c in (kc, vc):
        r = torch.full((w.B, w.Hkv, R, w.d), float("nan"), dtype=c.dtype, device=DEV)
        for b, L in enumerate(lens):
            pos = torch.arange(max(0, L - R), L, device=DEV)
            r[b, :, pos % R] = c[b, :, pos]
        rings.append(r)
    o_ring = sa.decode_ring(q, rings[0], rings[1], lens_t, mode="ssplit", seg=w.seg)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ring)
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens_t.cpu(), mode="ssplit", seg=w.seg)
    assert_close(o.float().cpu().numpy(), ref, "bf16", w.name)
