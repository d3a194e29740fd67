"""Maximum sizes: sequences of millions of positions, where byte offsets of a
(batch, head) slice approach 2^32 and positions need every bit of int32 index
arithmetic.  Sampled rows against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import Workload, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def prm(w):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def rows_of(N, rng, n=300):
    return np.unique(np.concatenate([rng.integers(0, N, n), [0, 1, 4095, N // 2, N - 2, N - 1]]))


@pytest.mark.parametrize("w", [
    # 2M positions, d = 128: a K slice is 512 MiB (byte offsets up to 2^29 per slice)
    Workload("max_window_d128", "window", "bf16", 1, 1, 1, 1 << 21, 128, k_win=512, scale_inputs=True, seed=161),
    # 1M positions with skip keys reaching 15 * 4096 back, and GQA
    Workload("max_pi_gqa", "pi", "bf16", 1, 2, 1, 1 << 20, 64, k_win=300, pi=4096, M=15, seed=162),
    Workload("max_ecp", "ecp", "bf16", 1, 1, 1, (1 << 20) + 77, 64, seg=2048, scale_inputs=True, seed=163),
], ids=lambda w: w.name)
def test_long_sequences_sampled(w):
    say("case %s" % (w,))
    q, k, v, a = prefill_inputs(w, device=DEV)
    o = sa.fwd(q, k, v, a, **prm(w))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    for h in range(w.Hq):
        rows = rows_of(w.N, rng) + h * w.N
        ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), None if a is None else a.cpu(), rows=rows, **prm(w))
        got = o.reshape(-1, w.d)[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
        assert_close(got, ref, "bf16", "%s head %d" % (w.name, h))


def test_long_cache_decode():
    # one sequence with a 2M-token cache, pi skips reaching 15 * 65536 back
    w = Workload("max_decode", "pi", "bf16", 2, 8, 2, 1 << 21, 128, k_win=1024, pi=65536, M=15, decode=True, seed=164)
    say("case %s" % (w,))
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens = torch.tensor([w.N, w.N - 12345], dtype=torch.int32, device=DEV)
    o = sa.decode(q, kc, vc, lens, a, **prm(w))
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens.cpu(), a.cpu(), **prm(w))
    assert_close(o.float().cpu().numpy(), ref, "bf16", w.name)


def test_long_sequence_backward():
    # window gradients are local: rows [s0, s0+R) need positions [s0-k, s0+R+k)
    from parity import assert_grad_close
    from structured_sparse_causal_amd.inputs import grad_output
    w = Workload("max_bwd", "window", "bf16", 1, 2, 1, 1 << 20, 64, k_win=700, seed=165)
    say("case %s" % (w,))
    q, k, v, _ = prefill_inputs(w, device=DEV)
    dO = grad_output(w, device=DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    o = sa.fwd(q, k, v, lse=lse, **prm(w))
    dq, dk, dv, _ = sa.bwd(q, k, v, None, o, lse, dO, **prm(w))
    torch.cuda.synchronize()
    K, R = w.k_win, 256
    for s0 in (0, w.N - R, 777777):
        lo, hi = max(0, s0 - K), min(w.N, s0 + R + K)
        sub = lambda t: t[:, :, lo:hi].cpu()
        rq, rk, rv, _ = oracle.bwd(sub(q), sub(k), sub(v), None, sub(dO), mode="window", k_win=K)
        r0 = s0 - lo
        got = lambda t: t[:, :, s0:s0 + R].float().cpu().numpy()
        assert_grad_close(got(dq), rq[:, :, r0:r0 + R], "dq rows %d" % s0)
        assert_grad_close(got(dk), rk[:, :, r0:r0 + R], "dk rows %d" % s0)
        assert_grad_close(got(dv), rv[:, :, r0:r0 + R], "dv rows %d" % s0)
