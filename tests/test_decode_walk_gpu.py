"""Decode with many (sequence, KV head, head chunk) workgroups: when they fill
at least three quarters of the compute units in their last round, each
workgroup walks all of its splits itself and writes the output directly (no
split partials, no combine).  These cases are sized to take that path on the
device they run on and compare it with the fp64 oracle, including lengths that
give NaN, unmapped pages, two head chunks per KV head, every mask mode that
decodes, d = 64 and d = 128, and the output gate."""
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


def walk_batch(Hkv, hchunks):
    """A batch whose workgroups fill all but a few compute units twice over."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B = 2 * cus // (Hkv * hchunks) - 1
    wgs = B * Hkv * hchunks
    assert 4 * wgs >= 3 * cus * -(-wgs // cus)
    return B


def ragged_lens(B, N, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, N + 1, B)
    lens[:4] = [1, 2, N, N - 1]
    return lens


def check(w, lens, o, q, kc, vc, a, sample, what):
    lens_t = torch.tensor(lens, dtype=torch.int32)
    for b in sample:
        ref = oracle.decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), lens_t[b:b + 1],
                            None if a is None or w.mode != "pi" else a[b:b + 1].cpu(), **prm(w))
        assert_close(o[b:b + 1].float().cpu().numpy(), ref, "bf16", "%s seq %d (len %d)" % (what, b, lens[b]))


CASES = [
    # (name, mode, Hq, Hkv, N, d, params); head chunks = ceil(Hq / Hkv / 16)
    ("pi_gqa4_d128", "pi", 16, 4, 700, 128, dict(k_win=100, pi=64, M=6)),
    ("pi_gqa32_d64", "pi", 64, 2, 500, 64, dict(k_win=300, pi=40, M=9)),
    ("window_d64", "window", 8, 8, 900, 64, dict(k_win=333)),
    ("ecp_d128", "ecp", 8, 2, 800, 128, dict(seg=96)),
    ("ssplit_d128", "ssplit", 8, 4, 600, 128, dict(seg=200)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_walk_decode_matches_oracle(case):
    name, mode, Hq, Hkv, N, d, p = case
    hchunks = -(-(Hq // Hkv) // 16)
    B = walk_batch(Hkv, hchunks)
    w = Workload(name, mode, "bf16", B, Hq, Hkv, N, d, decode=True, seed=300 + len(name), **p)
    say("walk %s B=%d" % (name, B))
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens = ragged_lens(B, N, w.seed)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = sa.decode(q, kc, vc, lens_t, a if mode == "pi" else None, **prm(w))
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    sample = sorted(set([0, 1, 2, 3, B - 1] + list(np.random.default_rng(1).integers(0, B, 12))))
    check(w, lens, o, q, kc, vc, a, sample, name)


def test_walk_decode_bad_lengths_and_pages():
    # lengths 0 and > Lmax give NaN rows (contiguous); an out-of-range table
    # entry gives NaN for that sequence only (paged, bit-equal elsewhere)
    Hq, Hkv, N, d, P = 16, 4, 640, 128, 32
    B = walk_batch(Hkv, 1)
    w = Workload("walk_bad", "pi", "bf16", B, Hq, Hkv, N, d, k_win=90, pi=50, M=8, decode=True, seed=321)
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens = ragged_lens(B, N, 5)
    bad = list(lens)
    bad[5], bad[6] = 0, N + 1
    o = sa.decode(q, kc, vc, torch.tensor(bad, dtype=torch.int32, device=DEV), a, **prm(w))
    ref = sa.decode(q, kc, vc, torch.tensor(lens, dtype=torch.int32, device=DEV), a, **prm(w))
    torch.cuda.synchronize()
    assert torch.isnan(o[5:7].float()).all()
    keep = [b for b in range(B) if b not in (5, 6)]
    assert torch.equal(o[keep], ref[keep])
    # paged copy of the same caches, pages at seeded random slots
    npg = N // P
    perm = torch.randperm(B * npg, generator=torch.Generator().manual_seed(7)).to(DEV)
    pools = []
    for c in (kc, vc):
        pool = torch.empty((B * npg, Hkv, P, d), dtype=c.dtype, device=DEV)
        pool[perm] = c.view(B, Hkv, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, P, d)
        pools.append(pool)
    table = perm.view(B, npg).to(torch.int32).contiguous()
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    op = sa.decode_paged(q, pools[0], pools[1], table, lens_t, a, **prm(w))
    torch.cuda.synchronize()
    assert torch.equal(op, ref)
    table[9, (int(lens[9]) - 1) // P] = B * npg        # the query's own page, out of range
    op = sa.decode_paged(q, pools[0], pools[1], table, lens_t, a, **prm(w))
    torch.cuda.synchronize()
    assert torch.isnan(op[9].float()).all()
    keep = [b for b in range(B) if b != 9]
    assert torch.equal(op[keep], ref[keep])
    check(w, lens, ref, q, kc, vc, a, [0, 3, 9, B - 1], "walk_bad")


def test_walk_decode_out_gate_and_ring():
    Hq, Hkv, N, d = 16, 4, 1000, 64
    B = walk_batch(Hkv, 1)
    w = Workload("walk_ring", "pi", "bf16", B, Hq, Hkv, N, d, k_win=120, pi=100, M=5, decode=True, seed=322)
    q, kc, vc, _, a = decode_inputs(w, device=DEV)
    lens = ragged_lens(B, N, 6)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ref = sa.decode(q, kc, vc, lens_t, a, **prm(w))
    R = max(w.k_win, w.M * w.pi) + 1
    rings = []
    for c in (kc, vc):
        r = torch.full((B, Hkv, R, d), float("nan"), dtype=c.dtype, device=DEV)
        for b, L in enumerate(lens):
            pos = torch.arange(max(0, int(L) - R), int(L), device=DEV)
            r[b, :, pos % R] = c[b, :, pos]
        rings.append(r)
    o = sa.decode_ring(q, rings[0], rings[1], lens_t, a, **prm(w))
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(8)).to(q.dtype)
    og = sa.decode(q, kc, vc, lens_t, a, out_gate=g.to(DEV), **prm(w))
    torch.cuda.synchronize()
    for b in (0, 2, B // 2, B - 1):
        r = oracle.decode(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), lens_t[b:b + 1].cpu(),
                          a[b:b + 1].cpu(), out_gate=g[b:b + 1], **prm(w))
        assert_close(og[b:b + 1].float().cpu().numpy(), r, "bf16", "walk out_gate seq %d" % b)
