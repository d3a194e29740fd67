"""Parity at full size, in the configurations the benchmark times beyond the
five workloads: the serving cache layouts and the fused options of the GQA
decode, the further mask modes, and the fused options of the prefill.  The
oracle computes sampled rows (or whole sequences) one by one; layouts that only
move rows are compared bit for bit with the contiguous decode."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import MASK_WORKLOADS, WORKLOADS, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def prm(w):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def sample_rows(rng, B, H, N, n):
    b = rng.integers(0, B, n)
    h = rng.integers(0, H, n)
    i = np.concatenate([rng.integers(0, N, n - 4), [0, 1, N - 1, N // 2]])
    return (b * H + h) * N + i


def test_decode_layouts_full_size():
    # the benchmark's decode_layouts leg: paged pools (16- and 64-row pages at
    # seeded random slots) and a ring of max(k, M*pi) + 1 rows
    w = WORKLOADS["decode_pi_gqa_bf16"]
    say("full-size decode layouts")
    q, kc, vc, lens, a = decode_inputs(w, device=DEV)
    ref = sa.decode(q, kc, vc, lens, a, **prm(w))
    B, H, L, d = kc.shape
    for P in (16, 64):
        npg = L // P
        gen = torch.Generator(device="cpu")
        gen.manual_seed(1000 + P)
        perm = torch.randperm(B * npg, generator=gen).to(DEV)
        pools = []
        for c in (kc, vc):
            pool = torch.empty((B * npg, H, P, d), dtype=c.dtype, device=DEV)
            pool[perm] = c.view(B, H, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, P, d)
            pools.append(pool)
        table = perm.view(B, npg).to(torch.int32).contiguous()
        o = sa.decode_paged(q, pools[0], pools[1], table, lens, a, **prm(w))
        torch.cuda.synchronize()
        assert torch.equal(o, ref), "paged P=%d" % P
        del pools
        torch.cuda.empty_cache()
    R = max(w.k_win, w.M * w.pi) + 1
    pos = torch.arange(L - R, L, device=DEV)
    rings = []
    for c in (kc, vc):
        r = torch.empty((B, H, R, d), dtype=c.dtype, device=DEV)
        r[:, :, pos % R] = c[:, :, pos]
        rings.append(r)
    o = sa.decode_ring(q, rings[0], rings[1], lens, a, **prm(w))
    torch.cuda.synchronize()
    assert torch.equal(o, ref), "ring"
    for b in (0, 40):
        r_or = oracle.decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), lens[b:b + 1].cpu(),
                             a[b:b + 1].cpu(), **prm(w))
        assert_close(ref[b:b + 1].float().cpu().numpy(), r_or, "bf16", "decode seq %d" % b)


@pytest.mark.parametrize("name", list(MASK_WORKLOADS))
def test_mask_modes_full_size_sampled(name):
    w = MASK_WORKLOADS[name]
    say("full-size %s" % name)
    q, k, v, _ = prefill_inputs(w, device=DEV)
    o = sa.fwd(q, k, v, **prm(w)).float().cpu().numpy().reshape(-1, w.d)
    rows = sample_rows(np.random.default_rng(9), w.B, w.Hq, w.N, 400 if w.d == 128 else 2000)
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), rows=rows, **prm(w))
    assert_close(o[rows], ref, "bf16", name)


def gate_params(w, gen):
    return ((0.5 * torch.randn((w.Hq, w.d), generator=gen) / math.sqrt(w.d)).float(),
            torch.randn((w.Hq,), generator=gen).float())


def test_fused_options_full_size_sampled():
    # the benchmark's fused_options leg: cosine scores and the output gate on
    # the ECP workload, the query-driven gate on the pi workload
    gen = torch.Generator().manual_seed(99)
    rng = np.random.default_rng(10)
    w = WORKLOADS["ecp_bf16"]
    q, k, v, _ = prefill_inputs(w, device=DEV)
    g = torch.randn(q.shape, generator=gen).to(q.dtype)
    rows = sample_rows(rng, w.B, w.Hq, w.N, 1500)
    for kw, okw, tag in ((dict(cosine=True, score_scale=10.0), dict(cosine=True, scale=10.0), "ecp cosine"),
                         (dict(out_gate=g.to(DEV)), dict(out_gate=g), "ecp out_gate")):
        say("full-size %s" % tag)
        o = sa.fwd(q, k, v, **prm(w), **kw).float().cpu().numpy().reshape(-1, w.d)
        ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), rows=rows, **prm(w), **okw)
        assert_close(o[rows], ref, "bf16", tag)
    del q, k, v, g
    w = WORKLOADS["pi_bf16"]
    say("full-size pi query gate")
    q, k, v, _ = prefill_inputs(w, device=DEV)
    gw, gb = gate_params(w, gen)
    o = sa.fwd(q, k, v, None, gate_w=gw.to(DEV), gate_b=gb.to(DEV), **prm(w)).float().cpu().numpy().reshape(-1, w.d)
    rows = sample_rows(rng, w.B, w.Hq, w.N, 1500)
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), None, rows=rows, gate_w=gw, gate_b=gb, **prm(w))
    assert_close(o[rows], ref, "bf16", "pi query gate")


def gate_mlp_params(w, H, gen):
    return ((torch.randn((w.Hq, H, w.d), generator=gen) / math.sqrt(w.d)).float(),
            (0.5 * torch.randn((w.Hq, H), generator=gen)).float(),
            (1.5 * torch.randn((w.Hq, H), generator=gen) / math.sqrt(H)).float(),
            (0.5 * torch.randn((w.Hq,), generator=gen)).float())


def test_pi_gate_network_full_size_sampled():
    # the benchmark's gate-network leg: the pi workload with alpha from the
    # two-layer gate (hidden width 32)
    w = WORKLOADS["pi_bf16"]
    say("full-size pi gate network")
    gen = torch.Generator().manual_seed(97)
    q, k, v, _ = prefill_inputs(w, device=DEV)
    w1, b1, w2, b2 = gate_mlp_params(w, 32, gen)
    o = sa.fwd(q, k, v, None, gate_w=w1.to(DEV), gate_b=b1.to(DEV), gate_w2=w2.to(DEV), gate_b2=b2.to(DEV),
               **prm(w)).float().cpu().numpy().reshape(-1, w.d)
    rows = sample_rows(np.random.default_rng(13), w.B, w.Hq, w.N, 4000)
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), None, rows=rows, gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2,
                     **prm(w))
    assert_close(o[rows], ref, "bf16", "pi gate network")


@pytest.mark.parametrize("network", [False, True], ids=["linear", "network"])
def test_pi_query_gate_several_chunks_sampled(network):
    # the query-driven gate with no alpha tensor, on a shape whose skip pass
    # and prefill run over several chunks of head groups
    w = WORKLOADS["pi_bf16"].replace(name="pi_gate_chunks", B=2, Hq=32, Hkv=8, N=32768, k_win=200, pi=700,
                                     M=20, seed=71)
    say("pi query gate (%s) over chunks %s" % ("network" if network else "linear", w))
    whole = w.B * w.Hq * w.N * (8 + 2 * w.d)
    assert 0 < sa.fwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, torch.bfloat16, "pi", w.k_win, w.pi,
                                    w.M) < whole / 2
    gen = torch.Generator().manual_seed(98)
    q, k, v, _ = prefill_inputs(w, device=DEV)
    if network:
        w1, b1, w2, b2 = gate_mlp_params(w, 20, gen)
        gk = dict(gate_w=w1, gate_b=b1, gate_w2=w2, gate_b2=b2)
    else:
        gw, gb = gate_params(w, gen)
        gk = dict(gate_w=gw, gate_b=gb)
    o = sa.fwd(q, k, v, None, **{key: t.to(DEV) for key, t in gk.items()}, **prm(w)).float().cpu().numpy()
    o = o.reshape(-1, w.d)
    rows = sample_rows(np.random.default_rng(12), w.B, w.Hq, w.N, 4000)
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), None, rows=rows, **gk, **prm(w))
    assert_close(o[rows], ref, "bf16", "pi query gate, chunked")


def test_decode_all_options_full_size():
    w = WORKLOADS["decode_pi_gqa_bf16"]
    say("full-size decode with every option")
    gen = torch.Generator().manual_seed(98)
    q, kc, vc, lens, _ = decode_inputs(w, device=DEV)
    gw, gb = gate_params(w, gen)
    og = torch.randn(q.shape, generator=gen).to(q.dtype)
    o = sa.decode(q, kc, vc, lens, None, cosine=True, score_scale=10.0, gate_w=gw.to(DEV), gate_b=gb.to(DEV),
                  out_gate=og.to(DEV), **prm(w))
    torch.cuda.synchronize()
    for b in (3, 63):
        ref = oracle.decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), lens[b:b + 1].cpu(), None,
                            cosine=True, scale=10.0, gate_w=gw, gate_b=gb, out_gate=og[b:b + 1], **prm(w))
        assert_close(o[b:b + 1].float().cpu().numpy(), ref, "bf16", "decode seq %d" % b)
