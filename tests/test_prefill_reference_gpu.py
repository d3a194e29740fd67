"""Prefill parity when the scores grow along the key axis.

The bf16 prefill takes the row max only on the first key tile a wave
computes; later tiles are checked against that reference and recompute their
scores and raise it when their probabilities would exceed 2^8 (or overflow).
Random inputs almost never reach that path, so these cases scale the key rows
up along the sequence (a ramp, and a late block of keys scaled far enough
that their probabilities against the first tile's reference overflow fp32):
every row must still match the fp64 oracle.
"""
from __future__ import annotations

import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import Workload, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def scaled_keys(k, gain):
    """k rows multiplied by gain[j] (fp32 product, rounded to k's dtype)."""
    g = torch.as_tensor(gain, dtype=torch.float32).view(1, 1, -1, 1)
    return (k.float() * g).to(k.dtype)


def ramp(N, top):
    return 1.0 + (top - 1.0) * torch.arange(N, dtype=torch.float32) / max(N - 1, 1)


def jump(N, at, factor):
    g = torch.ones(N, dtype=torch.float32)
    g[at:] = factor
    return g


CASES = [
    (Workload("ref_ecp_ramp", "ecp", "bf16", 1, 2, 2, 1536, 64, seg=256, seed=81), "ramp", 8.0),
    (Workload("ref_ecp_jump", "ecp", "bf16", 1, 2, 2, 1536, 64, seg=512, seed=82), "jump", 60.0),
    (Workload("ref_ssplit_ramp", "ssplit", "bf16", 1, 2, 2, 1100, 64, seg=300, seed=83), "ramp", 8.0),
    (Workload("ref_window_d128_ramp", "window", "bf16", 1, 2, 1, 1400, 128, k_win=700, seed=84), "ramp", 8.0),
    (Workload("ref_window_d128_jump", "window", "bf16", 1, 2, 2, 1000, 128, k_win=900, seed=85), "jump", 40.0),
    (Workload("ref_pi_ramp", "pi", "bf16", 1, 2, 2, 1300, 64, k_win=300, pi=128, M=6, seed=86), "ramp", 8.0),
    (Workload("ref_pi_jump", "pi", "bf16", 1, 2, 2, 1300, 64, k_win=500, pi=256, M=4, seed=87), "jump", 60.0),
]


@pytest.mark.parametrize("w,kind,amount", CASES, ids=lambda x: x.name if isinstance(x, Workload) else str(x))
def test_growing_scores(w, kind, amount):
    print("case %s %s %s" % (w, kind, amount), flush=True)
    q, k, v, a = prefill_inputs(w)
    gain = ramp(w.N, amount) if kind == "ramp" else jump(w.N, (2 * w.N) // 3, amount)
    k = scaled_keys(k, gain)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None if a is None else a.to(DEV), **prm)
    torch.cuda.synchronize()
    ref = oracle.fwd(q, k, v, a if w.mode == "pi" else None, **prm)
    assert_close(o.float().cpu().numpy(), ref, w.dtype, w.name)


def test_growing_scores_training_lse():
    """The row log-sum-exp written by the training forward follows the raised
    references too."""
    w = Workload("ref_lse_ecp_jump", "ecp", "bf16", 1, 2, 2, 1024, 64, seg=256, seed=88)
    q, k, v, a = prefill_inputs(w)
    k = scaled_keys(k, jump(w.N, 700, 50.0))
    lse = torch.empty(w.B, w.Hq, w.N, dtype=torch.float32, device=DEV)
    o = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), None, mode="ecp", seg=w.seg, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.fwd(q, k, v, None, mode="ecp", seg=w.seg)
    assert_close(o.float().cpu().numpy(), ref, "bf16", w.name)
    ref_lse = torch.as_tensor(oracle.lse(q, k, None, mode="ecp", seg=w.seg))
    err = float((lse.cpu().double() - ref_lse).abs().max())
    # lse reaches ~100 here; the kernel rounds each probability to bf16
    # (relative 2^-9) before summing, so allow that relative error of the sum
    assert err <= 1e-2, err
