"""Serving-cache decode (ring and paged KV caches) and graph replay on the GPU.

A ring or paged cache changes only where a position's row lives: the split
plan and the order of the rows are those of the contiguous decode, so the
outputs must equal the contiguous decode over the full cache bit for bit; they
are also compared with the fp64 oracle.  Cache slots and pages that hold no
written position are filled with NaN, so reading one shows up in the output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import structured_sparse_causal_amd as sa
from parity import assert_close
from structured_sparse_causal_amd.inputs import Workload, decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def prm(w: Workload):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def full_inputs(w: Workload, lens):
    """Contiguous caches [B, Hkv, N, d] on the GPU (N = w.N >= max(lens))."""
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, kc, vc, lens_t, a


def to_ring(cache, lens, R):
    B, H, _, d = cache.shape
    ring = torch.full((B, H, R, d), float("nan"), dtype=cache.dtype, device=cache.device)
    for b, L in enumerate(lens):
        pos = torch.arange(max(0, L - R), L, device=cache.device)
        ring[b, :, pos % R] = cache[b, :, pos]
    return ring


def to_paged(kc, vc, lens, P, rng, spare=7):
    """Pools [num_pages, Hkv, P, d] with the pages of every sequence at random
    physical positions, the block table [B, max_pages] (-1 = unmapped)."""
    B, H, N, d = kc.shape
    max_pages = -(-N // P)
    need = [-(-L // P) for L in lens]
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    kp = torch.full((num_pages, H, P, d), float("nan"), dtype=kc.dtype, device=kc.device)
    vp = torch.full_like(kp, float("nan"))
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    at = 0
    for b, L in enumerate(lens):
        for j in range(need[b]):
            page = int(perm[at])
            at += 1
            table[b, j] = page
            n = min(P, L - j * P)
            kp[page, :, :n] = kc[b, :, j * P:j * P + n]
            vp[page, :, :n] = vc[b, :, j * P:j * P + n]
    return kp, vp, table.to(kc.device), num_pages


def contiguous(q, kc, vc, lens_t, a, w):
    o = sa.decode(q, kc, vc, lens_t, a if w.mode == "pi" else None, **prm(w))
    torch.cuda.synchronize()
    return o


def oracle_check(o, q, kc, vc, lens_t, a, w, what):
    ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens_t.cpu(), None if a is None or w.mode != "pi" else a.cpu(),
                        **prm(w))
    assert_close(o.float().cpu().numpy(), ref, "bf16", what)


RING_CASES = [
    # (workload, lens, R); R >= the key span (k + 1, M*pi + 1, 2*seg)
    (Workload("ring_pi", "pi", "bf16", 4, 8, 2, 4321, 128, k_win=64, pi=50, M=4, decode=True, seed=91),
     [150, 201, 1000, 4321], 201),
    (Workload("ring_pi_gqa4_d64", "pi", "bf16", 3, 16, 4, 3000, 64, k_win=300, pi=128, M=15, decode=True, seed=92),
     [1, 2000, 3000], 1921),
    (Workload("ring_window", "window", "bf16", 3, 8, 8, 2500, 128, k_win=100, decode=True, seed=93),
     [101, 102, 2500], 101),
    (Workload("ring_ecp", "ecp", "bf16", 3, 4, 1, 1800, 128, seg=64, decode=True, seed=94),
     [64, 129, 1799], 128),
]


@pytest.mark.parametrize("w,lens,R", RING_CASES, ids=[c[0].name for c in RING_CASES])
def test_ring_decode(w, lens, R):
    say("ring %s lens %s R %d" % (w.name, lens, R))
    q, kc, vc, lens_t, a = full_inputs(w, lens)
    ref = contiguous(q, kc, vc, lens_t, a, w)
    kr, vr = to_ring(kc, lens, R), to_ring(vc, lens, R)
    o = sa.decode_ring(q, kr, vr, lens_t, a if w.mode == "pi" else None, **prm(w))
    torch.cuda.synchronize()
    assert torch.equal(o, ref), "ring decode differs from the contiguous decode"
    oracle_check(o, q, kc, vc, lens_t, a, w, w.name)


PAGED_CASES = [
    (Workload("paged_pi_gqa8", "pi", "bf16", 5, 32, 8, 3000, 128, k_win=200, pi=128, M=15, decode=True, seed=95),
     [1, 17, 64, 1000, 3000], 16),
    (Workload("paged_pi_p64", "pi", "bf16", 4, 8, 2, 5000, 128, k_win=512, pi=300, M=12, decode=True, seed=96),
     [700, 4097, 4999, 5000], 64),
    (Workload("paged_window_d64", "window", "bf16", 3, 8, 8, 2000, 64, k_win=333, decode=True, seed=97),
     [1, 334, 2000], 32),
    (Workload("paged_ecp", "ecp", "bf16", 3, 4, 2, 1500, 128, seg=100, decode=True, seed=98),
     [99, 700, 1500], 8),
]


@pytest.mark.parametrize("w,lens,P", PAGED_CASES, ids=[c[0].name for c in PAGED_CASES])
def test_paged_decode(w, lens, P):
    say("paged %s lens %s P %d" % (w.name, lens, P))
    q, kc, vc, lens_t, a = full_inputs(w, lens)
    ref = contiguous(q, kc, vc, lens_t, a, w)
    kp, vp, table, _ = to_paged(kc, vc, lens, P, np.random.default_rng(w.seed))
    o = sa.decode_paged(q, kp, vp, table, lens_t, a if w.mode == "pi" else None, **prm(w))
    torch.cuda.synchronize()
    assert torch.equal(o, ref), "paged decode differs from the contiguous decode"
    oracle_check(o, q, kc, vc, lens_t, a, w, w.name)


def test_paged_unmapped_page_gives_nan_for_that_sequence_only():
    w, lens, P = PAGED_CASES[0]
    q, kc, vc, lens_t, a = full_inputs(w, lens)
    ref = contiguous(q, kc, vc, lens_t, a, w)
    kp, vp, table, num_pages = to_paged(kc, vc, lens, P, np.random.default_rng(3))
    table[3, (lens[3] - 1) // P] = num_pages          # the query's own page, out of range
    table[4, 0] = -5                                  # a page no key of sequence 4 needs
    o = sa.decode_paged(q, kp, vp, table, lens_t, a, **prm(w))
    torch.cuda.synchronize()
    assert torch.isnan(o[3].float()).all()
    keep = [0, 1, 2, 4]
    assert torch.equal(o[keep], ref[keep])


def test_paged_decode_graph_replay():
    """A captured paged decode replayed with new queries, lengths and block
    tables written into its input buffers between replays, with eager work and
    synchronisation in between; every replay equals the eager call."""
    w, lens, P = PAGED_CASES[0]
    q, kc, vc, lens_t, a = full_inputs(w, lens)
    kp, vp, table, _ = to_paged(kc, vc, lens, P, np.random.default_rng(11))
    out = torch.empty_like(q)
    nbytes = sa.binding.load_library().sparse_attn_decode_paged_workspace_size(
        w.B, w.Hq, w.Hkv, P, table.shape[1], w.d, 1, 0, w.k_win, w.pi, w.M, w.seg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    call = lambda o: sa.decode_paged(q, kp, vp, table, lens_t, a, out=o, workspace=ws, **prm(w))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    rng = np.random.default_rng(12)
    mapped = [(b, j) for b in range(w.B) for j in range(-(-lens[b] // P))]
    for rep in range(4):
        q.copy_(torch.randn(q.shape, device=DEV).to(q.dtype))
        # shorter lengths (their pages stay mapped) ...
        lens_t.copy_(torch.tensor([int(rng.integers(1, L + 1)) for L in lens], dtype=torch.int32))
        # ... and two physical pages swapped, contents and table entries together
        (b1, j1), (b2, j2) = [mapped[i] for i in rng.choice(len(mapped), 2, replace=False)]
        p1, p2 = int(table[b1, j1]), int(table[b2, j2])
        kp[[p1, p2]] = kp[[p2, p1]]
        vp[[p1, p2]] = vp[[p2, p1]]
        table[b1, j1], table[b2, j2] = p2, p1
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = torch.empty_like(out)
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager call" % rep
        ref = contiguous(q, kc, vc, lens_t, a, w)
        assert torch.equal(out, ref), "replay %d differs from the contiguous decode" % rep
