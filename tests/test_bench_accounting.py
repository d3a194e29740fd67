"""The benchmark's useful-work accounting (CPU).

bench.py reports useful TFLOP/s = 4*d FLOP per attended (query, key) pair and
useful bytes = one read of q, k, v (and alpha) plus one write of o.  These
tests pin its pair counts to the oracle's own key-set enumeration on small
shapes (every mask mode) and to closed forms at the benchmark's workloads:
window pairs (k+1)(k+2)/2 + (N-k-1)(k+1) for N > k, skip pairs
pi * sum_p min(M, p) when pi > k and N = P*pi, ECP pairs
s(s+1)/2 + (C-1)(s^2 + s(s+1)/2) for N = C*s.
"""
from __future__ import annotations

import pytest

import bench
import oracle
from structured_sparse_causal_amd.inputs import WORKLOADS, Workload

SMALL = [
    Workload("a_pi", "pi", "bf16", 1, 1, 1, 97, 64, k_win=9, pi=13, M=5),
    Workload("a_pi_overlap", "pi", "bf16", 1, 1, 1, 80, 64, k_win=20, pi=6, M=7),
    Workload("a_pi_pi1", "pi", "bf16", 1, 1, 1, 40, 64, k_win=3, pi=1, M=9),
    Workload("a_window", "window", "bf16", 1, 1, 1, 77, 64, k_win=12),
    Workload("a_window_dense", "window", "bf16", 1, 1, 1, 33, 64, k_win=500),
    Workload("a_ecp", "ecp", "bf16", 1, 1, 1, 70, 64, seg=9),
    Workload("a_ecp_s1", "ecp", "bf16", 1, 1, 1, 20, 64, seg=1),
    Workload("a_bidir", "window_bidir", "bf16", 1, 1, 1, 61, 64, k_win=7),
    Workload("a_ssplit", "ssplit", "bf16", 1, 1, 1, 59, 64, seg=11),
    Workload("a_ecp_full", "ecp_full", "bf16", 1, 1, 1, 65, 64, seg=8),
]


def _oracle_pairs(w: Workload) -> int:
    return sum(len(oracle.key_set(i, w.mode, w.k_win, w.pi, w.M, w.seg, N=w.N)[0]) for i in range(w.N))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_pairs_match_oracle_key_sets(w):
    assert bench.pairs_per_head(w) == _oracle_pairs(w)


@pytest.mark.parametrize("L", [1, 2, 50, 300, 1000])
def test_decode_keys_match_oracle(L):
    w = Workload("a_dec", "pi", "bf16", 1, 1, 1, L, 64, k_win=40, pi=30, M=6, decode=True)
    keys, _ = oracle.key_set(L - 1, "pi", w.k_win, w.pi, w.M, 0, N=L)
    assert bench.decode_keys(w, L) == len(keys)


def _window_pairs(N, k):
    return (k + 1) * (k + 2) // 2 + (N - k - 1) * (k + 1)


def test_closed_forms_at_the_benchmark_workloads():
    c1, c2, c3 = WORKLOADS["pi_tiny_f32"], WORKLOADS["ecp_bf16"], WORKLOADS["pi_bf16"]
    c4, c5 = WORKLOADS["window_loop_bf16"], WORKLOADS["decode_pi_gqa_bf16"]
    # tiny pi-Attention: window 7,920 plus skips 64 * (0+1+2+3) = 384
    assert _window_pairs(256, 32) == 7920
    assert bench.pairs_per_head(c1) == 7920 + 64 * (0 + 1 + 2 + 3)
    # ECP, s = 512, 8 half-segments
    s, C = 512, 8
    assert bench.pairs_per_head(c2) == s * (s + 1) // 2 + (C - 1) * (s * s + s * (s + 1) // 2) == 2885632
    # pi-Attention: window 4,177,792 plus skips 1024 * (0+1+...+15) = 122,880
    assert bench.pairs_per_head(c3) == _window_pairs(16384, 256) + 1024 * sum(min(15, p) for p in range(16))
    assert bench.pairs_per_head(c3) == 4300672
    # looped window: 66,649,600 per (batch, head) and call
    assert bench.pairs_per_head(c4) == _window_pairs(65536, 1024) == 66649600
    # decode: 2,049 window keys plus 14 skip keys below the window
    assert bench.decode_keys(c5, c5.N) == 2063


def test_useful_flop_and_bytes():
    w = WORKLOADS["ecp_bf16"]
    flop, nbytes = bench.prefill_useful(w)
    assert flop == 4 * 64 * 2885632 * 4 * 12
    assert nbytes == 2 * 64 * 4096 * 4 * 12 * 4          # q, k, v, o in bf16
    w = WORKLOADS["pi_bf16"]
    _, nbytes = bench.prefill_useful(w)
    assert nbytes == 2 * 64 * 16384 * 2 * 16 * 4 + 4 * 2 * 16 * 16384   # plus alpha (fp32)
    w = WORKLOADS["decode_pi_gqa_bf16"]
    flop, nbytes = bench.decode_useful(w)
    assert nbytes == 541860096                             # attended cache rows, q, o, alpha, lens
    assert flop == 4 * 128 * 2063 * 64 * 32
