"""The prefill forward (with the pi skip pass and its workspace), the looped
block and a training step (forward with lse, then the backward) captured in
HIP graphs and replayed with new inputs written into the captured buffers,
with eager work and synchronisation between replays: every replay equals
the eager call bit for bit.  The library allocates nothing and issues no
memset, so its launches are capturable; the binding's output and workspace
tensors come from the graph's memory pool."""
from __future__ import annotations

import torch
import pytest

import structured_sparse_causal_amd as sa
from structured_sparse_causal_amd.inputs import Workload, grad_output, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def capture(fn):
    """Warm up on a side stream, then capture fn() in a graph; returns (graph, outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def refill(*ts):
    for t in ts:
        if t is None:
            continue
        if t.dtype == torch.float32 and t.dim() == 3:       # alpha in (0, 1)
            t.copy_(torch.sigmoid(torch.randn(t.shape, device=DEV)))
        else:
            t.copy_(torch.randn(t.shape, device=DEV).to(t.dtype))


@pytest.mark.parametrize("w", [
    Workload("gr_pi_skips", "pi", "bf16", 1, 4, 2, 1500, 64, k_win=100, pi=128, M=5, seed=191),
    Workload("gr_ecp_d128", "ecp", "bf16", 2, 2, 2, 1024, 128, seg=128, seed=192),
], ids=lambda w: w.name)
def test_prefill_graph_replay(w):
    q, k, v, a = [t.to(DEV) if t is not None else None for t in prefill_inputs(w)]
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    g, o = capture(lambda: sa.fwd(q, k, v, a, lse=lse, **prm(w)))
    for rep in range(3):
        refill(q, k, v, a)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lse_e = torch.empty_like(lse)
        o_e = sa.fwd(q, k, v, a, lse=lse_e, **prm(w))
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), "%s replay %d: o differs from the eager call" % (w.name, rep)
        assert torch.equal(lse, lse_e), "%s replay %d: lse differs from the eager call" % (w.name, rep)


def test_looped_block_graph_replay():
    w = Workload("gr_loop", "window", "bf16", 1, 4, 4, 4096, 128, k_win=512, seed=193)
    q, k, v, _ = [t.to(DEV) if t is not None else None for t in prefill_inputs(w)]
    g, o = capture(lambda: sa.loop_fwd(q, k, v, steps=4, mode="window", k_win=w.k_win))
    for rep in range(3):
        refill(q, k, v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e = sa.loop_fwd(q, k, v, steps=4, mode="window", k_win=w.k_win)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), "replay %d differs from the eager looped block" % rep


def test_training_step_graph_replay():
    w = Workload("gr_train_pi", "pi", "bf16", 1, 4, 2, 1200, 64, k_win=90, pi=100, M=6, seed=194)
    q, k, v, a = [t.to(DEV) for t in prefill_inputs(w)]
    dO = grad_output(w).to(DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)

    def step():
        o = sa.fwd(q, k, v, a, lse=lse, **prm(w))
        return (o,) + tuple(sa.bwd(q, k, v, a, o, lse, dO, **prm(w)))

    g, outs = capture(step)
    for rep in range(3):
        refill(q, k, v, a, dO)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = step()
        torch.cuda.synchronize()
        for name, x, y in zip(("o", "dq", "dk", "dv", "dalpha"), outs, eager):
            assert torch.equal(x, y), "replay %d: %s differs from the eager step" % (rep, name)
