"""Pins of the fp64 CPU oracle against facts fixed by the pages and by
mathematics, independent of the oracle's own code (CPU only).

Each pin is chosen to catch a plausible mistake: a dropped or wrong-signed
prior, a prior indexed by key instead of query, an off-by-one window or
half-segment bound, a skip counted twice, a transposed operand, a wrong GQA
head map or a wrong scale.
"""
from __future__ import annotations

import glob
import math
import os

import numpy as np
import pytest
import torch

import oracle
from parity import gate_failures
from structured_sparse_causal_amd.inputs import WORKLOADS, prefill_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent dense construction: the mask comes from an arithmetic predicate
# over the distance i - j, evaluated on whole index grids (no key lists).
# ---------------------------------------------------------------------------
def predicate_bias(N, mode, k_win=0, pi=0, M=0, seg=0, alpha_row=None):
    """Additive bias [N, N] for one head: log-prior on attended pairs, -inf
    elsewhere.  alpha_row [N] is the gate of each query row (PI only)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    dist = i - j
    bias = np.full((N, N), -np.inf)
    if mode == "ecp":
        vis = (dist >= 0) & ((j // seg) >= (i // seg) - 1)
        bias[vis] = 0.0
        return bias
    local = (dist >= 0) & (dist <= k_win)
    if mode == "window":
        bias[local] = 0.0
        return bias
    a = np.asarray(alpha_row, dtype=np.float64)[:, None] * np.ones((1, N))
    skip = np.zeros((N, N), dtype=bool)
    if M > 0:
        skip = (dist > k_win) & (dist % pi == 0) & (dist // pi >= 1) & (dist // pi <= M)
    with np.errstate(divide="ignore"):
        bias[local] = np.log(a[local])
        bias[skip] = np.log1p(-a[skip])
    return bias


def dense_attention(q, k, v, bias):
    """softmax(q k^T / sqrt(d) + bias) v in fp64 for one head; q,k,v [N,d]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = q @ k.T / math.sqrt(q.shape[1]) + bias
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def randn(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).numpy()


def rand_alpha(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.sigmoid(torch.randn(shape, generator=g, dtype=torch.float32)).numpy()


# ---------------------------------------------------------------------------
# Worked examples (closed forms derived by hand in tests/golden/*.txt)
# ---------------------------------------------------------------------------
def _read_golden(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "e*.txt"))),
                         ids=lambda p: os.path.basename(p))
def test_worked_example(path):
    g = _read_golden(path)
    N, d = int(g["N"][0]), 4
    mode = g["mode"][0]
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    v = np.repeat(np.arange(N, dtype=np.float32)[:, None], d, axis=1)[None, None]
    alpha = np.full((1, 1, N), float(g["alpha"][0]), np.float32)
    o = oracle.fwd(q, k, v, alpha if mode == "pi" else None, mode=mode,
                   k_win=int(g["k_win"][0]), pi=int(g["pi"][0]), M=int(g["M"][0]),
                   seg=int(g["seg"][0]))
    expected = np.array([float(x) for x in g["expected"]])
    for c in range(d):
        np.testing.assert_allclose(o[0, 0, :, c], expected, rtol=0, atol=1e-12)


def test_e2_rejects_multiset_reading():
    """The overlap example separates the set reading from a multiset one."""
    g = _read_golden(os.path.join(GOLDEN, "e2_pi_overlap.txt"))
    multiset = np.array([0, 0.5, 0.5, 1.5, 5 / 3, 8 / 3, 2.75, 3.75])
    assert np.abs(np.array([float(x) for x in g["expected"]]) - multiset).max() > 0.4


# ---------------------------------------------------------------------------
# Key sets: brute force against the distance predicate
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["pi", "window", "ecp"])
def test_key_set_bruteforce(mode):
    N = 70
    grid = []
    if mode == "ecp":
        grid = [dict(seg=s) for s in (1, 2, 3, 7, 16, 64, 100)]
    elif mode == "window":
        grid = [dict(k_win=kk) for kk in (0, 1, 5, 31, 69, 200)]
    else:
        grid = [dict(k_win=kk, pi=p, M=m) for kk in (0, 1, 4, 9) for p in (1, 2, 3, 5, 8, 13)
                for m in (0, 1, 3, 20)]
    for prm in grid:
        kw = dict(k_win=0, pi=0, M=0, seg=0)
        kw.update(prm)
        bias = predicate_bias(N, mode, alpha_row=np.full(N, 0.5), **kw)
        for i in range(N):
            keys, labels = oracle.key_set(i, mode, **kw)
            assert list(keys) == sorted(set(keys.tolist())), "keys must be distinct and ascending"
            expect = set(np.nonzero(np.isfinite(bias[i]))[0].tolist())
            assert set(keys.tolist()) == expect, (mode, prm, i)
            if mode == "pi":
                for j, lab in zip(keys, labels):
                    assert lab == (0 if i - j <= kw["k_win"] else 1), (prm, i, j)


def test_key_counts_of_workloads():
    """Per-query key counts quoted for the workloads (window 257 keys plus up to
    15 skips; decode query at 32767 sees 2049 + 14 keys)."""
    keys, lab = oracle.key_set(16383, "pi", k_win=256, pi=1024, M=15)
    assert len(keys) == 257 + 15 and int((lab == 1).sum()) == 15
    keys, lab = oracle.key_set(32767, "pi", k_win=2048, pi=2048, M=15)
    assert len(keys) == 2063 and int((lab == 1).sum()) == 14
    keys, _ = oracle.key_set(4095, "ecp", seg=512)
    assert len(keys) == 1024
    keys, _ = oracle.key_set(100, "window", k_win=1024)
    assert len(keys) == 101


# ---------------------------------------------------------------------------
# Reductions to dense attention
# ---------------------------------------------------------------------------
def test_window_wide_equals_dense_causal_sdpa():
    """k >= N-1 and no skips: dense causal softmax attention (torch SDPA, fp64)."""
    B, H, N, d = 2, 3, 40, 16
    q, k, v = randn((B, H, N, d), 1), randn((B, H, N, d), 2), randn((B, H, N, d), 3)
    o = oracle.fwd(q, k, v, mode="window", k_win=N + 5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(),
        torch.from_numpy(v).double(), is_causal=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("prm", [dict(k_win=5, pi=7, M=4), dict(k_win=3, pi=2, M=6),
                                 dict(k_win=0, pi=1, M=9), dict(k_win=8, pi=9, M=1),
                                 dict(k_win=12, pi=5, M=0)])
def test_pi_equals_dense_with_predicate_bias(prm):
    B, Hq, Hkv, N, d = 1, 4, 2, 48, 8
    q, k, v = randn((B, Hq, N, d), 11), randn((B, Hkv, N, d), 12), randn((B, Hkv, N, d), 13)
    alpha = rand_alpha((B, Hq, N), 14)
    o = oracle.fwd(q, k, v, alpha, mode="pi", **prm)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        bias = predicate_bias(N, "pi", alpha_row=alpha[0, h], **prm)
        ref = dense_attention(q[0, h], k[0, g], v[0, g], bias)
        np.testing.assert_allclose(o[0, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seg", [1, 4, 5, 16, 47, 64])
def test_ecp_equals_dense_with_pair_mask(seg):
    B, H, N, d = 1, 2, 47, 8
    q, k, v = randn((B, H, N, d), 21), randn((B, H, N, d), 22), randn((B, H, N, d), 23)
    o = oracle.fwd(q, k, v, mode="ecp", seg=seg)
    for h in range(H):
        ref = dense_attention(q[0, h], k[0, h], v[0, h], predicate_bias(N, "ecp", seg=seg))
        np.testing.assert_allclose(o[0, h], ref, rtol=0, atol=1e-12)


def test_ecp_special_cases():
    """s >= N is dense causal; s = 1 leaves keys {i-1, i}."""
    B, H, N, d = 1, 1, 20, 4
    q, k, v = randn((B, H, N, d), 31), randn((B, H, N, d), 32), randn((B, H, N, d), 33)
    dense = oracle.fwd(q, k, v, mode="window", k_win=N)
    np.testing.assert_allclose(oracle.fwd(q, k, v, mode="ecp", seg=N), dense, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.fwd(q, k, v, mode="ecp", seg=1),
                               oracle.fwd(q, k, v, mode="window", k_win=1), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Invariants and closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode,prm", [("pi", dict(k_win=4, pi=6, M=3)),
                                      ("window", dict(k_win=9)), ("ecp", dict(seg=8))])
def test_rows_sum_to_one(mode, prm):
    B, H, N, d = 1, 2, 64, 8
    q, k = randn((B, H, N, d), 41), randn((B, H, N, d), 42)
    v = np.ones((B, H, N, d), np.float32)
    alpha = rand_alpha((B, H, N), 43) if mode == "pi" else None
    o = oracle.fwd(q, k, v, alpha, mode=mode, **prm)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_explicit_probabilities_closed_form():
    """Q = K = 0 and V = I: output rows are the probability rows, which are
    alpha_i / (alpha_i nW + (1-alpha_i) nS) on the window of i and
    (1-alpha_i) / (...) on its skips -- with alpha taken from the QUERY row."""
    N = d = 32
    prm = dict(k_win=3, pi=5, M=4)
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    v = np.eye(N, d, dtype=np.float32)[None, None]
    alpha = rand_alpha((1, 1, N), 51)
    p = oracle.fwd(q, k, v, alpha, mode="pi", **prm)[0, 0]
    for i in range(N):
        a = float(alpha[0, 0, i])
        win = [j for j in range(max(0, i - 3), i + 1)]
        skp = [i - m * 5 for m in range(1, 5) if i - m * 5 >= 0 and m * 5 > 3]
        z = a * len(win) + (1 - a) * len(skp)
        expect = np.zeros(N)
        expect[win] = a / z
        expect[skp] = (1 - a) / z
        np.testing.assert_allclose(p[i], expect, rtol=0, atol=1e-7)


def test_alpha_one_equals_window_bitwise():
    B, H, N, d = 1, 2, 80, 8
    q, k, v = randn((B, H, N, d), 61), randn((B, H, N, d), 62), randn((B, H, N, d), 63)
    ones = np.ones((B, H, N), np.float32)
    a = oracle.fwd(q, k, v, ones, mode="pi", k_win=6, pi=10, M=5)
    b = oracle.fwd(q, k, v, mode="window", k_win=6)
    assert np.array_equal(a, b)


def test_alpha_near_one_difference_is_order_eps():
    B, H, N, d = 1, 1, 80, 8
    q, k, v = randn((B, H, N, d), 64), randn((B, H, N, d), 65), randn((B, H, N, d), 66)
    win = oracle.fwd(q, k, v, mode="window", k_win=6)
    diffs = []
    for eps in (1e-2, 1e-3, 1e-4):
        a = np.full((B, H, N), 1 - eps, np.float32)
        o = oracle.fwd(q, k, v, a, mode="pi", k_win=6, pi=10, M=5)
        diffs.append(np.abs(o - win).max())
    assert diffs[0] > 0
    assert diffs[1] < diffs[0] / 5 and diffs[2] < diffs[1] / 5


def test_rows_without_skips_ignore_alpha():
    B, H, N, d = 1, 1, 60, 8
    q, k, v = randn((B, H, N, d), 71), randn((B, H, N, d), 72), randn((B, H, N, d), 73)
    prm = dict(k_win=5, pi=20, M=2)
    o1 = oracle.fwd(q, k, v, rand_alpha((B, H, N), 74), mode="pi", **prm)
    o2 = oracle.fwd(q, k, v, rand_alpha((B, H, N), 75), mode="pi", **prm)
    rows_without = [i for i in range(N) if i < 20]   # i - 20 < 0: no skip key
    rows_with = [i for i in range(N) if i >= 20]
    np.testing.assert_allclose(o1[0, 0, rows_without], o2[0, 0, rows_without], rtol=0, atol=1e-13)
    assert np.abs(o1[0, 0, rows_with] - o2[0, 0, rows_with]).max() > 1e-3


def test_zero_window_is_identity_bitwise():
    B, H, N, d = 1, 2, 30, 8
    q, k, v = randn((B, H, N, d), 81), randn((B, H, N, d), 82), randn((B, H, N, d), 83)
    o = oracle.fwd(q, k, v, mode="window", k_win=0)
    assert np.array_equal(o, v.astype(np.float64))
    o = oracle.fwd(q, k, v, np.full((B, H, N), 0.3, np.float32), mode="pi", k_win=0, pi=3, M=0)
    assert np.array_equal(o, v.astype(np.float64))


def test_softmax_scale_is_inv_sqrt_d():
    """Two keys only (window k=1, row 1): p(key 0) = sigmoid((s0 - s1)/sqrt(d))."""
    d = 16
    q = randn((1, 1, 2, d), 91)
    k = randn((1, 1, 2, d), 92)
    v = np.zeros((1, 1, 2, d), np.float32)
    v[0, 0, 0, :] = 1.0
    o = oracle.fwd(q, k, v, mode="window", k_win=1)
    s0 = float(np.dot(q[0, 0, 1].astype(np.float64), k[0, 0, 0]))
    s1 = float(np.dot(q[0, 0, 1].astype(np.float64), k[0, 0, 1]))
    assert abs(o[0, 0, 1, 0] - 1 / (1 + math.exp((s1 - s0) / 4.0))) < 1e-14


def test_loop_cone_bitwise():
    """After T applications of a window-k block with the output fed back as V,
    row i depends only on V rows [i - T k, i] ("LT2", section 2.2: receptive
    field O(T w))."""
    B, H, N, d, kw, T = 1, 2, 96, 8, 5, 3
    q, k, v = randn((B, H, N, d), 101), randn((B, H, N, d), 102), randn((B, H, N, d), 103)
    base = oracle.loop_fwd(q, k, v, steps=T, mode="window", k_win=kw)
    v2 = v.copy()
    i0 = 60
    v2[:, :, : i0 - T * kw] += randn(v2[:, :, : i0 - T * kw].shape, 104) * 10
    pert = oracle.loop_fwd(q, k, v2, steps=T, mode="window", k_win=kw)
    assert np.array_equal(base[-1][:, :, i0:], pert[-1][:, :, i0:])
    assert not np.array_equal(base[-1][:, :, i0 - 1], pert[-1][:, :, i0 - 1])


def test_decode_equals_prefill_row():
    B, Hq, Hkv, L, d = 3, 4, 2, 50, 8
    prm = dict(k_win=6, pi=7, M=4)
    q = randn((B, Hq, L, d), 111)
    k, v = randn((B, Hkv, L, d), 112), randn((B, Hkv, L, d), 113)
    alpha = rand_alpha((B, Hq, L), 114)
    full = oracle.fwd(q, k, v, alpha, mode="pi", **prm)
    lens = np.array([50, 17, 1], np.int32)
    qd = np.stack([q[b, :, lens[b] - 1] for b in range(B)])
    ad = np.stack([alpha[b, :, lens[b] - 1] for b in range(B)])
    od = oracle.decode(qd, k, v, lens, ad, mode="pi", **prm)
    for b in range(B):
        np.testing.assert_allclose(od[b], full[b, :, lens[b] - 1], rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, N, d = 2, 6, 2, 40, 8
    prm = dict(k_win=4, pi=9, M=3)
    q = randn((B, Hq, N, d), 121)
    k, v = randn((B, Hkv, N, d), 122), randn((B, Hkv, N, d), 123)
    alpha = rand_alpha((B, Hq, N), 124)
    o = oracle.fwd(q, k, v, alpha, mode="pi", **prm)
    rep = Hq // Hkv
    o2 = oracle.fwd(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), alpha,
                    mode="pi", **prm)
    assert np.array_equal(o, o2)


def test_selected_rows_match_full():
    w = WORKLOADS["pi_tiny_f32"]
    q, k, v, a = prefill_inputs(w)
    full = oracle.fwd(q, k, v, a, mode="pi", k_win=w.k_win, pi=w.pi, M=w.M)
    rows = np.array([0, 5, 255, 256 + 100, 511])
    sel = oracle.fwd(q, k, v, a, mode="pi", k_win=w.k_win, pi=w.pi, M=w.M, rows=rows)
    np.testing.assert_array_equal(sel, full.reshape(-1, w.d)[rows])


def test_alpha_domain_is_checked():
    q = np.zeros((1, 1, 4, 4), np.float32)
    for bad in (0.0, -0.5, 1.5, float("nan")):
        a = np.full((1, 1, 4), bad, np.float32)
        with pytest.raises(ValueError):
            oracle.fwd(q, q, q, a, mode="pi", k_win=1, pi=2, M=1)


def test_round_to_bf16_matches_rne():
    """fp64 -> bf16 rounding: on fp32-representable values it must equal the
    float32 -> bfloat16 round-to-nearest-even conversion; hand-made ties go to
    the even neighbour."""
    x = randn((10000,), 131).astype(np.float64) * 37.0
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x), ref)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6).
    got = oracle.round_to_bf16(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8) - 1e-12]))
    np.testing.assert_array_equal(got, [1.0, 1 + 2 ** -6, -(1 + 2 ** -7)])


# ---------------------------------------------------------------------------
# The comparison gates catch wrong outputs that the absolute bounds alone miss
# ---------------------------------------------------------------------------
def test_gates_reject_zeros_and_wrong_masks():
    B, H, N, d = 1, 2, 256, 32
    g = torch.Generator().manual_seed(7)
    q = (torch.randn((B, H, N, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    k = (torch.randn((B, H, N, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    v = (torch.randn((B, H, N, d), generator=g) / math.sqrt(d)).to(torch.bfloat16)
    ref = oracle.fwd(q, k, v, mode="ecp", seg=32)
    bf = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert gate_failures(bf, ref, "bf16") == []          # a faithful bf16 output passes
    assert gate_failures(np.zeros_like(ref), ref, "bf16") != []
    # ECP whose queries also see half-segment c-2
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    far = np.where((j <= i) & ((j // 32) >= (i // 32) - 2), 0.0, -np.inf)
    wrong = np.stack([dense_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                      v[0, h].float().numpy(), far) for h in range(H)])[None]
    assert gate_failures(wrong, ref, "bf16") != []
    wref = oracle.fwd(q, k, v, mode="window", k_win=64)
    assert gate_failures(oracle.fwd(q, k, v, mode="window", k_win=63), wref, "bf16") != []


def test_loop_closed_form_window_means():
    """The looped block (LT2 page, section 1 and section 2.2) with Q = K = 0:
    every application is a plain mean over the window, so with V[j, :] = j
    the rows follow by hand.  Rows i <= k see [0, i] at every step:
    O_1[i] = i/2, and inductively O_T[i] = i / 2^T.  Rows i >= T k see only
    rows that are at least (T-1) k: O_1[i] = i - k/2, and inductively
    O_T[i] = i - T k / 2.  All values are exact in bf16 here, so the rounded
    feedback (V_{t+1} = bf16(O_t)) changes nothing."""
    N, d, kw, T = 48, 4, 4, 4
    q = np.zeros((1, 1, N, d), np.float32)
    v = np.repeat(np.arange(N, dtype=np.float32)[None, None, :, None], d, axis=3)
    outs = oracle.loop_fwd(q, q, v, steps=T, mode="window", k_win=kw)
    assert len(outs) == T
    i = np.arange(N, dtype=np.float64)
    for t, o in enumerate(outs, start=1):
        col = o[0, 0, :, 0]
        assert np.array_equal(o, np.repeat(col[:, None], d, axis=1)[None, None])
        assert np.array_equal(col[: kw + 1], i[: kw + 1] / 2.0 ** t)
        assert np.array_equal(col[t * kw:], i[t * kw:] - t * kw / 2.0)
    # a dropped feedback (V fixed) would give i - k/2 at every step
    assert not np.array_equal(outs[-1][0, 0, T * kw:, 0], i[T * kw:] - kw / 2.0)
