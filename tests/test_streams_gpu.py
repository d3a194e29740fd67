"""Calls on several streams at once (each with its own outputs and
workspace) give the results of the same calls made one after another: the
library keeps no state between calls, so concurrent calls on different
streams do not interfere.  (The allocation-free decode, which shares one
device scratch per GPU, is the documented exception and is not used here.)"""
from __future__ import annotations

import pytest
import torch

import structured_sparse_causal_amd as sa
from structured_sparse_causal_amd.inputs import Workload, decode_inputs, grad_output, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def test_concurrent_streams_match_sequential():
    wp = Workload("st_pi", "pi", "bf16", 1, 4, 2, 2000, 64, k_win=128, pi=160, M=6, seed=195)
    we = Workload("st_ecp", "ecp", "bf16", 2, 4, 4, 2048, 128, seg=256, seed=196)
    wd = Workload("st_dec", "pi", "bf16", 8, 16, 4, 4000, 128, k_win=512, pi=512, M=7, decode=True, seed=197)
    pi_in = [t.to(DEV) for t in prefill_inputs(wp)]
    ecp_in = [t.to(DEV) if t is not None else None for t in prefill_inputs(we)]
    dO = grad_output(wp).to(DEV)
    dq, dkc, dvc, lens, da = [t.to(DEV) for t in decode_inputs(wd)]

    def run_pi():
        q, k, v, a = pi_in
        lse = torch.empty((wp.B, wp.Hq, wp.N), dtype=torch.float32, device=DEV)
        o = sa.fwd(q, k, v, a, lse=lse, **prm(wp))
        return (o, lse) + tuple(sa.bwd(q, k, v, a, o, lse, dO, **prm(wp)))

    def run_ecp():
        q, k, v, _ = ecp_in
        return (sa.loop_fwd(q, k, v, steps=2, **prm(we)),)

    def run_dec():
        return (sa.decode(dq, dkc, dvc, lens, da, **prm(wd)),)

    seq = [f() for f in (run_pi, run_ecp, run_dec)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = [None] * 3
        for i, (s, f) in enumerate(zip(streams, (run_pi, run_ecp, run_dec))):
            with torch.cuda.stream(s):
                got[i] = f()
        torch.cuda.synchronize()
        for i, (a_res, b_res) in enumerate(zip(seq, got)):
            for j, (x, y) in enumerate(zip(a_res, b_res)):
                assert torch.equal(x, y), "rep %d call %d result %d differs from the sequential run" % (rep, i, j)
