"""Pins for the oracle's further mask modes (CPU only).

    window_bidir  j in [i-k, i+k]              (the window as the pi-Attention page states it)
    ssplit        j in [floor(i/s)*s, i]       (s-Split segments of the ECP page, causal)
    ecp_full      j in half-segments c-1, c    (the ECP PAR block without the causal mask)

Each is pinned against something that does not share the oracle's key-set
code: torch's scaled_dot_product_attention where the mask reduces to dense
(causal or not), exact identities, the reversal symmetry of the two-sided
window, per-segment reductions to dense attention on slices, a vectorised
distance-predicate mask, and torch autograd through that dense form.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


def predicate_mask(N, mode, k_win=0, seg=0):
    """[N, N] boolean visibility from arithmetic on positions only."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if mode == "window_bidir":
        return np.abs(i - j) <= k_win
    if mode == "ssplit":
        return (i // seg == j // seg) & (j <= i)
    if mode == "ecp_full":
        return (i // seg - j // seg >= 0) & (i // seg - j // seg <= 1)
    raise ValueError(mode)


def dense(q, k, v, mask):
    s = q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(q.shape[-1])
    s = np.where(mask, s, -np.inf)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v.astype(np.float64)


def sdpa(q, k, v, causal):
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal).numpy()


MODES = [dict(mode="window_bidir", k_win=5), dict(mode="window_bidir", k_win=0),
         dict(mode="ssplit", seg=6), dict(mode="ssplit", seg=1), dict(mode="ecp_full", seg=5),
         dict(mode="ecp_full", seg=1)]


@pytest.mark.parametrize("prm", MODES, ids=lambda p: "-".join("%s%s" % kv for kv in p.items()))
def test_key_sets_match_predicate(prm):
    N = 37
    mask = predicate_mask(N, **prm)
    for i in range(N):
        keys, labels = oracle.key_set(i, N=N, **prm)
        assert list(keys) == list(np.nonzero(mask[i])[0])
        assert (labels == 0).all()


@pytest.mark.parametrize("prm", MODES, ids=lambda p: "-".join("%s%s" % kv for kv in p.items()))
def test_equals_dense_with_predicate_mask(prm):
    B, H, N, d = 1, 2, 41, 16
    q, k, v = rnd((B, H, N, d), 1), rnd((B, H, N, d), 2), rnd((B, H, N, d), 3)
    o = oracle.fwd(q, k, v, **prm)
    for h in range(H):
        ref = dense(q[0, h], k[0, h], v[0, h], predicate_mask(N, **prm))
        assert np.abs(o[0, h] - ref).max() < 1e-12


def test_wide_masks_reduce_to_sdpa():
    B, H, N, d = 1, 3, 29, 8
    q, k, v = rnd((B, H, N, d), 4), rnd((B, H, N, d), 5), rnd((B, H, N, d), 6)
    full = sdpa(q, k, v, causal=False)
    causal = sdpa(q, k, v, causal=True)
    assert np.abs(oracle.fwd(q, k, v, mode="window_bidir", k_win=N) - full).max() < 1e-12
    assert np.abs(oracle.fwd(q, k, v, mode="ecp_full", seg=N) - full).max() < 1e-12
    assert np.abs(oracle.fwd(q, k, v, mode="ssplit", seg=N) - causal).max() < 1e-12


def test_identities():
    # k = 0 and s = 1 leave each query with only itself: o = v exactly.
    q, k, v = rnd((1, 2, 19, 8), 7), rnd((1, 2, 19, 8), 8), rnd((1, 2, 19, 8), 9)
    for prm in (dict(mode="window_bidir", k_win=0), dict(mode="ssplit", seg=1)):
        assert np.array_equal(oracle.fwd(q, k, v, **prm), v.astype(np.float64))


def test_bidirectional_window_is_reversal_symmetric():
    # [i-k, i+k] maps onto itself when positions are reversed, so reversing
    # the sequence reverses the output.
    q, k, v = rnd((1, 2, 33, 8), 10), rnd((1, 2, 33, 8), 11), rnd((1, 2, 33, 8), 12)
    o = oracle.fwd(q, k, v, mode="window_bidir", k_win=4)
    rev = lambda x: np.ascontiguousarray(x[:, :, ::-1])
    o_r = oracle.fwd(rev(q), rev(k), rev(v), mode="window_bidir", k_win=4)
    assert np.abs(rev(o_r) - o).max() < 1e-12


def test_segment_reductions():
    # s-Split: segment c is causal attention over its own rows only;
    # ecp_full: half-segment c is unmasked attention of its queries over the
    # rows of half-segments c-1 and c.
    B, H, N, d, s = 1, 2, 30, 8, 7
    q, k, v = rnd((B, H, N, d), 13), rnd((B, H, N, d), 14), rnd((B, H, N, d), 15)
    o_split = oracle.fwd(q, k, v, mode="ssplit", seg=s)
    o_full = oracle.fwd(q, k, v, mode="ecp_full", seg=s)
    for c in range(0, (N + s - 1) // s):
        a, e = c * s, min(N, (c + 1) * s)
        ref = sdpa(q[:, :, a:e], k[:, :, a:e], v[:, :, a:e], causal=True)
        assert np.abs(o_split[:, :, a:e] - ref).max() < 1e-12
        lo = max(0, (c - 1) * s)
        t = lambda x: torch.tensor(x, dtype=torch.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q[:, :, a:e]), t(k[:, :, lo:e]), t(v[:, :, lo:e])).numpy()
        assert np.abs(o_full[:, :, a:e] - ref).max() < 1e-12


@pytest.mark.parametrize("prm", MODES[::2], ids=lambda p: p["mode"])
def test_bwd_matches_autograd(prm):
    B, Hq, Hkv, N, d = 1, 4, 2, 23, 8
    q, k, v = rnd((B, Hq, N, d), 16), rnd((B, Hkv, N, d), 17), rnd((B, Hkv, N, d), 18)
    dO = rnd((B, Hq, N, d), 19)
    dq, dk, dv, _ = oracle.bwd(q, k, v, None, dO, **prm)
    mask = torch.tensor(predicate_mask(N, **prm))
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kr, vr = kt.repeat_interleave(Hq // Hkv, 1), vt.repeat_interleave(Hq // Hkv, 1)
    s = qt @ kr.transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(~mask, -math.inf)
    o = torch.softmax(s, dim=-1) @ vr
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    for got, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.abs(got - ref.numpy()).max() < 1e-10 * max(1.0, ref.abs().max().item())


def test_decode_rejects_noncausal_modes():
    q = rnd((1, 1, 8), 20)
    c = rnd((1, 1, 16, 8), 21)
    lens = np.array([16], dtype=np.int32)
    for prm in (dict(mode="window_bidir", k_win=3), dict(mode="ecp_full", seg=4)):
        with pytest.raises(ValueError):
            oracle.decode(q, c, c, lens, **prm)
    # s-Split is causal: decode equals the last prefill row
    qf = rnd((1, 1, 16, 8), 22)
    full = oracle.fwd(qf, c, c, mode="ssplit", seg=5)
    dec = oracle.decode(np.ascontiguousarray(qf[:, :, 15]), c, c, lens, mode="ssplit", seg=5)
    assert np.abs(dec - full[:, :, 15]).max() < 1e-12
