"""Prefill parity on seeded random shapes and mask parameters.

Ninety-six configurations drawn once from a fixed seed: every mask mode,
d = 64 and 128, bf16 and fp32, GQA ratios 1-4, sequence lengths that are not
multiples of the 128-row query blocks or the key tiles, windows and segments
of any size (including wider than the sequence) and skip periods below and
above the window.  Every output element is compared with the fp64 oracle.
Forty-eight more (bf16) run the training forward and the backward and compare
every gradient element with the oracle's fp64 chain rule, and forty-eight
decode cases with ragged cache lengths compare every output element.

SA_RANDOM_SHAPES="seed,n_fwd,n_bwd,n_dec" draws other (or more) cases from the
same generators: the seed is added to each generator's own, the counts replace
96, 48 and 48.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import Workload, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MODES = ["pi", "window", "ecp", "window_bidir", "ssplit", "ecp_full"]
_draw = [int(x) for x in os.environ.get("SA_RANDOM_SHAPES", "0,96,48,48").split(",")]
SEED_SHIFT, N_FWD, N_BWD, N_DEC = _draw


def _cases(n=N_FWD, seed=2024 + SEED_SHIFT):
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        mode = MODES[idx % len(MODES)]
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        hkv = int(rng.integers(1, 3))
        hq = hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.integers(1, 1400))
        k_win = int(rng.integers(0, max(2, N + 100)))
        seg = int(rng.integers(1, max(2, N // 2 + 64)))
        pi = int(rng.integers(1, max(2, N // 3 + 2)))
        M = int(rng.integers(0, 12)) if mode == "pi" else 0
        out.append(Workload("rand%02d_%s_%s_d%d" % (idx, mode, dtype, d), mode, dtype, B, hq, hkv, N, d,
                            k_win=k_win, pi=pi, M=M, seg=seg, scale_inputs=bool(rng.random() < 0.5),
                            seed=500 + idx + SEED_SHIFT))
    return out


@pytest.mark.parametrize("w", _cases(), ids=lambda w: w.name)
def test_random_shape(w):
    print("case %s" % (w,), flush=True)
    q, k, v, a = prefill_inputs(w)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if a is None else a.to(DEV), **prm)
    torch.cuda.synchronize()
    ref = oracle.fwd(q, k, v, a if w.mode == "pi" else None, **prm)
    assert_close(o.float().cpu().numpy(), ref, w.dtype, w.name)


def _bwd_cases(n=N_BWD, seed=4048 + SEED_SHIFT):
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        mode = MODES[idx % len(MODES)]
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 3))
        hq = hkv * int(rng.choice([1, 2, 4]))
        N = int(rng.integers(2, 900))
        out.append(Workload("rbwd%02d_%s_d%d" % (idx, mode, d), mode, "bf16", 1, hq, hkv, N, d,
                            k_win=int(rng.integers(0, N + 50)), pi=int(rng.integers(1, max(2, N // 3 + 2))),
                            M=int(rng.integers(0, 10)) if mode == "pi" else 0,
                            seg=int(rng.integers(1, max(2, N // 2 + 64))), seed=700 + idx + SEED_SHIFT))
    return out


@pytest.mark.parametrize("w", _bwd_cases(), ids=lambda w: w.name)
def test_random_shape_backward(w):
    """Gradients (dq, dk, dv, dalpha) of the training forward + backward on
    random shapes, against the oracle's fp64 chain rule."""
    from parity import assert_grad_close
    from structured_sparse_causal_amd.inputs import grad_output
    print("case %s" % (w,), flush=True)
    q, k, v, a = prefill_inputs(w)
    dO = grad_output(w)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    ad = None if a is None else a.to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    o = sa.fwd(qd, kd, vd, ad, lse=lse, **prm)
    dq, dk, dv, da = sa.bwd(qd, kd, vd, ad, o, lse, dO.to(DEV), **prm)
    torch.cuda.synchronize()
    a_or = a if w.mode == "pi" else None
    rq, rk, rv, ra = oracle.bwd(q, k, v, a_or, dO, **prm)
    assert_grad_close(dq.float().cpu().numpy(), rq, w.name + " dq")
    assert_grad_close(dk.float().cpu().numpy(), rk, w.name + " dk")
    assert_grad_close(dv.float().cpu().numpy(), rv, w.name + " dv")
    if w.mode == "pi":
        assert_grad_close(da.cpu().numpy(), ra, w.name + " dalpha")


def _decode_cases(n=N_DEC, seed=8096 + SEED_SHIFT):
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        mode = ["pi", "window", "ecp", "ssplit"][idx % 4]
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 5))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(1, 3000))
        out.append(Workload("rdec%02d_%s_d%d" % (idx, mode, d), mode, "bf16", int(rng.integers(1, 40)), hq, hkv, L,
                            d, k_win=int(rng.integers(0, L + 50)), pi=int(rng.integers(1, max(2, L // 3 + 2))),
                            M=int(rng.integers(0, 16)) if mode == "pi" else 0,
                            seg=int(rng.integers(1, max(2, L // 2 + 64))), decode=True, seed=900 + idx + SEED_SHIFT))
    return out


@pytest.mark.parametrize("w", _decode_cases(), ids=lambda w: w.name)
def test_random_shape_decode(w):
    """Single-token decode with ragged cache lengths (1..L per sequence) on
    random shapes; the batch sizes span both the split plan and the walk
    schedule."""
    from structured_sparse_causal_amd.inputs import decode_inputs
    print("case %s" % (w,), flush=True)
    q, kc, vc, lens, a = decode_inputs(w)
    g = torch.Generator().manual_seed(w.seed)
    lens = torch.randint(1, w.N + 1, (w.B,), generator=g, dtype=torch.int32)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    o = sa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), None if a is None else a.to(DEV), **prm)
    torch.cuda.synchronize()
    ref = oracle.decode(q, kc, vc, lens, a if w.mode == "pi" else None, **prm)
    assert_close(o.float().cpu().numpy(), ref, "bf16", w.name)
