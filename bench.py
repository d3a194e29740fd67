"""Benchmark of the causal structured-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One "step" is one pass of the headline workload (default: the looped
window-attention block, bf16, B=1 H=32 N=65536 d=128, window k=1024, applied
4 times with each output fed back as the next V: the largest single-GPU
configuration) on synthetic inputs already resident in HBM.  ``value`` is
useful TFLOP/s: 4*d FLOPs per attended (query, key) pair, nothing for masked
or padded work.  The same JSON line carries the roofline of the dominant
kernel (timed live with HIP events on the launch stream), a cold-cache timing
of the step, the other workloads of the hot path (ECP, pi-Attention prefill,
the fp32 tiny case, GQA decode) each with its own roofline fraction and
recorded HBM traffic, the backward pass of one layer call on the three
prefill shapes, and the CPU oracle timed on a bounded sample of the headline
workload.

Only one GPU is used; ``--gpus N`` with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 (published)
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
METRIC = "useful TFLOP/s + % bf16 MFMA peak (prefill); decode HBM GB/s (1 GPU)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "structured_sparse_causal_amd/csrc/"
# Sources whose kernels a workload's library call runs: a recorded counter
# measurement is reused only while their hash is unchanged.
_PREFILL_SOURCES = (_CSRC + "prefill.hip", _CSRC + "common.hpp", _CSRC + "kernels.hpp")
KERNEL_SOURCES = {
    "prefill": _PREFILL_SOURCES,
    "pi": _PREFILL_SOURCES + (_CSRC + "skip.hip", _CSRC + "api.hip"),
    "decode": (_CSRC + "decode.hip", _CSRC + "common.hpp", _CSRC + "kernels.hpp", _CSRC + "api.hip"),
}


def source_set(w) -> str:
    if w.decode:
        return "decode"
    return "pi" if (w.mode == "pi" and w.M > 0) else "prefill"


def kernel_source_hash(kind: str = "prefill") -> str:
    """sha256 over the sources of the kernels one call of that kind runs."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(w, key: str = "hbm_bytes_per_launch"):
    """HBM bytes of the workload's dominant kernel per launch (or, with
    key="hbm_bytes_per_call", of every kernel of one library call), from the
    rocprofv3 counter summary committed under profiles/ (FETCH_SIZE and
    WRITE_SIZE, each scaled by the reading of a plain copy of known size).
    None if there is no summary for this workload or its kernels changed
    since it was taken."""
    path = os.path.join(PROFILES, "counters_%s.md" % w.name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash(source_set(w)):
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def dominant_kernel(w) -> str:
    if w.decode:
        return "decode_bf16_kernel<%d, ...>" % w.d
    if w.dtype == "f32":
        return "prefill_f32_kernel<%d>" % w.d
    return "prefill_bf16_kernel<%d, %d>" % (w.d, 64 if w.d == 64 else 32)   # <head dim, key-tile rows>


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: %d copies of %d bytes" % (reps, nbytes))


# ---------------------------------------------------------------------------
# Useful work (attended pairs) and algorithmic bytes, from the mask definitions
# ---------------------------------------------------------------------------
def key_lo(i, w):
    if w.mode in ("ecp", "ecp_full"):
        return np.maximum(0, (i // w.seg - 1) * w.seg)
    if w.mode == "ssplit":
        return (i // w.seg) * w.seg
    return np.maximum(0, i - w.k_win)


def key_hi(i, w, N):
    if w.mode == "window_bidir":
        return np.minimum(N - 1, i + w.k_win)
    if w.mode == "ecp_full":
        return np.minimum(N - 1, (i // w.seg + 1) * w.seg - 1)
    return i


def pairs_per_head(w, N=None):
    """Attended (query, key) pairs of one (batch, head): window or ECP range
    plus, for pi-Attention, the skip keys lying below the window."""
    N = w.N if N is None else N
    i = np.arange(N, dtype=np.int64)
    n = (key_hi(i, w, N) - key_lo(i, w) + 1).sum()
    if w.mode == "pi" and w.M > 0:
        lo = key_lo(i, w)
        for m in range(1, w.M + 1):
            j = i - m * w.pi
            n += int(((j >= 0) & (j < lo)).sum())
    return int(n)


def decode_keys(w, L):
    i = L - 1
    lo = int(key_lo(np.array([i]), w)[0])
    n = i - lo + 1
    if w.mode == "pi":
        n += sum(1 for m in range(1, w.M + 1) if 0 <= i - m * w.pi < lo)
    return n


def prefill_useful(w):
    flop = 4.0 * w.d * pairs_per_head(w) * w.B * w.Hq
    es = 2 if w.dtype == "bf16" else 4
    nbytes = es * w.d * w.N * (2 * w.B * w.Hq + 2 * w.B * w.Hkv)
    if w.mode == "pi":
        nbytes += 4 * w.B * w.Hq * w.N
    return flop, float(nbytes)


def decode_useful(w):
    keys = decode_keys(w, w.N)
    es = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.Hkv * keys
    nbytes = 2 * rows * w.d * es + 2 * w.B * w.Hq * w.d * es + 4 * w.B
    if w.mode == "pi":
        nbytes += 4 * w.B * w.Hq
    flop = 4.0 * w.d * keys * w.B * w.Hq
    return flop, float(nbytes)


# ---------------------------------------------------------------------------
# Timing helpers
# ---------------------------------------------------------------------------
def event_times(torch, fn, reps):
    """Per-call GPU durations (ms) from HIP events recorded on the current
    stream, the stream the library launches on."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def warm(torch, fn, calls, seconds=0.15):
    """Untimed calls: at least ``calls``, and until ``seconds`` of GPU work have
    passed, so the clock has risen before anything is timed."""
    t0 = time.perf_counter()
    n = 0
    while n < calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def run_prefill_workload(torch, sa, w, reps, warmup):
    from structured_sparse_causal_amd.inputs import prefill_inputs
    dev = torch.device("cuda:0")
    q, k, v, a = prefill_inputs(w, device=dev)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    outs = (torch.empty_like(q), torch.empty_like(q))
    nbytes = sa.fwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, w.mode, w.k_win, w.pi,
                                   w.M, w.seg)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if w.loops > 1:
        def fn():
            sa.loop_fwd(q, k, v, a, steps=w.loops, outs=outs, workspace=ws, **prm)
    else:
        def fn():
            sa.fwd(q, k, v, a, out=outs[0], workspace=ws, **prm)
    warm(torch, fn, warmup)
    t = event_times(torch, fn, reps)
    flop, nb = prefill_useful(w)
    flop *= w.loops
    nb *= w.loops
    ms = float(np.median(t))
    ai = flop / nb
    attainable = min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1000.0)
    res = {
        "ms": ms, "ms_p10": float(np.percentile(t, 10)), "ms_p90": float(np.percentile(t, 90)),
        "useful_tflops": flop / (ms * 1e-3) / 1e12,
        "pct_bf16_mfma_peak": 100.0 * flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "arith_intensity": ai, "attainable_tflops": attainable,
        "pct_attainable": 100.0 * flop / (ms * 1e-3) / 1e12 / attainable,
        "useful_flop": flop, "useful_bytes": nb, "launches": w.loops * (2 if nbytes else 1),
    }
    res.update(workload_roofline(w, flop, nb, ms / max(w.loops, 1)))
    del q, k, v, a, outs, ws
    return res


def workload_roofline(w, flop, nb, ms_call):
    """Roofline fraction of one library call of the workload (all its
    kernels) and the HBM bytes recorded for that call under profiles/."""
    per_call_flop, per_call_bytes = flop / max(w.loops, 1), nb / max(w.loops, 1)
    if w.decode:
        bound, frac = "hbm", per_call_bytes / (ms_call * 1e-3) / 1e9 / HBM_PEAK_GBS
    elif w.dtype == "f32":
        bound, frac = "mfma_f32", per_call_flop / (ms_call * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS
    else:
        attainable = min(MFMA_BF16_PEAK_TFLOPS, per_call_flop / per_call_bytes * HBM_PEAK_GBS / 1000.0)
        bound = "mfma" if attainable >= MFMA_BF16_PEAK_TFLOPS else "hbm"
        frac = per_call_flop / (ms_call * 1e-3) / 1e12 / attainable
    t = recorded_traffic(w, "hbm_bytes_per_call")
    return {"bound": bound, "frac": frac, "traffic": t,
            "traffic_over_algorithmic": (t / per_call_bytes) if t is not None else None,
            "dominant_kernel": dominant_kernel(w)}


def run_decode_workload(torch, sa, w, reps, warmup):
    from structured_sparse_causal_amd.inputs import decode_inputs
    dev = torch.device("cuda:0")
    q, kc, vc, lens, a = decode_inputs(w, device=dev)
    out = torch.empty_like(q)
    nbytes = sa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, w.mode, w.k_win, w.pi,
                                      w.M, w.seg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def fn():
        sa.decode(q, kc, vc, lens, a, mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg,
                  out=out, workspace=ws)
    warm(torch, fn, warmup)
    t = event_times(torch, fn, reps)
    flop, nb = decode_useful(w)
    ms = float(np.median(t))
    res = {
        "ms": ms, "ms_p10": float(np.percentile(t, 10)), "ms_p90": float(np.percentile(t, 90)),
        "useful_GBps": nb / (ms * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "tokens_per_s": w.B / (ms * 1e-3), "useful_bytes": nb, "useful_flop": flop,
    }
    res.update(workload_roofline(w, flop, nb, ms))
    del q, kc, vc, lens, a, out, ws
    return res


def run_decode_layouts(torch, sa, w, reps, warmup):
    """The decode workload over serving-cache layouts holding the same rows:
    paged pools (page size 16 and 64, pages at seeded random physical slots)
    and a ring of max(k_win, M*pi) + 1 rows.  Same algorithmic bytes as the
    contiguous decode; the paged call also reads its block-table entries."""
    from structured_sparse_causal_amd.inputs import decode_inputs
    dev = torch.device("cuda:0")
    q, kc, vc, lens, a = decode_inputs(w, device=dev)
    _, nb = decode_useful(w)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    out = torch.empty_like(q)
    res = {}

    def timed(fn):
        warm(torch, fn, warmup)
        t = event_times(torch, fn, reps)
        ms = float(np.median(t))
        return {"ms": ms, "useful_GBps": nb / (ms * 1e-3) / 1e9,
                "pct_hbm_peak": 100.0 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "tokens_per_s": w.B / (ms * 1e-3)}

    B, H, L, d = kc.shape
    for P in (16, 64):
        npg = L // P
        gen = torch.Generator(device="cpu")
        gen.manual_seed(1000 + P)
        perm = torch.randperm(B * npg, generator=gen).to(dev)
        pools = []
        for c in (kc, vc):
            pool = torch.empty((B * npg, H, P, d), dtype=c.dtype, device=dev)
            pool[perm] = c.view(B, H, npg, P, d).permute(0, 2, 1, 3, 4).reshape(B * npg, H, P, d)
            pools.append(pool)
        table = perm.view(B, npg).to(torch.int32).contiguous()
        nbytes = sa.binding.load_library().sparse_attn_decode_paged_workspace_size(
            B, w.Hq, H, P, npg, d, 1, sa.binding._mode(w.mode), w.k_win, w.pi, w.M, w.seg)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        res["paged_p%d" % P] = timed(lambda: sa.decode_paged(q, pools[0], pools[1], table, lens, a, out=out,
                                                            workspace=ws, **prm))
        del pools, table, ws
        torch.cuda.empty_cache()
    R = max(w.k_win, w.M * w.pi if w.mode == "pi" else 0) + 1
    pos = torch.arange(L - R, L, device=dev)
    rings = []
    for c in (kc, vc):
        r = torch.empty((B, H, R, d), dtype=c.dtype, device=dev)
        r[:, :, pos % R] = c[:, :, pos]
        rings.append(r)
    res["ring_R%d" % R] = timed(lambda: sa.decode_ring(q, rings[0], rings[1], lens, a, out=out, **prm))
    del q, kc, vc, lens, a, rings, out
    return res


def run_option_workloads(torch, sa, reps, warmup):
    """Fused gate and epilogue options at the benchmark shapes, each timed
    against the plain call on the same inputs (same useful FLOP or bytes):
    cosine scores (ECP), the query-driven gate (pi-Attention: one layer, and
    the two-layer network of hidden width 32), the output
    gate (ECP), and all three in the GQA decode."""
    from structured_sparse_causal_amd.inputs import WORKLOADS, decode_inputs, prefill_inputs
    dev = torch.device("cuda:0")
    res = {}

    def timed(fn):
        warm(torch, fn, warmup)
        return float(np.median(event_times(torch, fn, reps)))

    gen = torch.Generator(device="cpu")
    gen.manual_seed(99)
    for name, wname, opt in (("ecp_cosine", "ecp_bf16", "cosine"), ("pi_query_gate", "pi_bf16", "gate"),
                             ("pi_gate_network_h32", "pi_bf16", "network"), ("ecp_out_gate", "ecp_bf16", "out_gate")):
        w = WORKLOADS[wname]
        q, k, v, a = prefill_inputs(w, device=dev)
        prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
        out = torch.empty_like(q)
        kw = {}
        if opt == "cosine":
            kw = dict(cosine=True, score_scale=10.0)
        elif opt == "gate":
            kw = dict(gate_w=(0.5 * torch.randn((w.Hq, w.d), generator=gen) / math.sqrt(w.d)).to(dev),
                      gate_b=torch.randn((w.Hq,), generator=gen).to(dev))
        elif opt == "network":   # two layers, ReLU hidden layer of width 32
            kw = dict(gate_w=(torch.randn((w.Hq, 32, w.d), generator=gen) / math.sqrt(w.d)).to(dev),
                      gate_b=(0.5 * torch.randn((w.Hq, 32), generator=gen)).to(dev),
                      gate_w2=(1.5 * torch.randn((w.Hq, 32), generator=gen) / math.sqrt(32)).to(dev),
                      gate_b2=(0.5 * torch.randn((w.Hq,), generator=gen)).to(dev))
        else:
            kw = dict(out_gate=torch.randn(q.shape, generator=gen).to(q.dtype).to(dev))
        alpha = None if opt in ("gate", "network") else a
        ms_plain = timed(lambda: sa.fwd(q, k, v, a, out=out, **prm))
        ms_opt = timed(lambda: sa.fwd(q, k, v, alpha, out=out, **prm, **kw))
        flop, _ = prefill_useful(w)
        res[name] = {"ms": ms_opt, "ms_plain": ms_plain, "useful_tflops": flop / (ms_opt * 1e-3) / 1e12,
                     "overhead_pct": 100.0 * (ms_opt / ms_plain - 1.0)}
        del q, k, v, a, out, kw
        torch.cuda.empty_cache()
    w = WORKLOADS["decode_pi_gqa_bf16"]
    q, kc, vc, lens, a = decode_inputs(w, device=dev)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    out = torch.empty_like(q)
    kw = dict(cosine=True, score_scale=10.0,
              gate_w=(0.5 * torch.randn((w.Hq, w.d), generator=gen) / math.sqrt(w.d)).to(dev),
              gate_b=torch.randn((w.Hq,), generator=gen).to(dev),
              out_gate=torch.randn(q.shape, generator=gen).to(q.dtype).to(dev))
    ms_plain = timed(lambda: sa.decode(q, kc, vc, lens, a, out=out, **prm))
    ms_opt = timed(lambda: sa.decode(q, kc, vc, lens, None, out=out, **prm, **kw))
    _, nb = decode_useful(w)
    res["decode_all_options"] = {"ms": ms_opt, "ms_plain": ms_plain, "useful_GBps": nb / (ms_opt * 1e-3) / 1e9,
                                 "overhead_pct": 100.0 * (ms_opt / ms_plain - 1.0)}
    del q, kc, vc, lens, a, out, kw
    return res


def run_bwd_workload(torch, sa, w, reps, warmup):
    """Backward pass of one layer call (bf16): gradients of q, k, v (and
    alpha) given dO, from the o and lse of a training forward run before the
    timed region.  Useful FLOP = 10*d per attended pair: the five contractions
    of the standard attention backward (recomputed scores, dP, dV, dK, dQ,
    2*d each), i.e. 2.5 times the forward's useful FLOP."""
    from structured_sparse_causal_amd.inputs import grad_output, prefill_inputs
    dev = torch.device("cuda:0")
    q, k, v, a = prefill_inputs(w, device=dev)
    dO = grad_output(w, device=dev)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    o = sa.fwd(q, k, v, a, lse=lse, **prm)
    nbytes = sa.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, w.mode, w.k_win, w.pi,
                                   w.M, w.seg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def fn():
        sa.bwd(q, k, v, a, o, lse, dO, workspace=ws, **prm)
    warm(torch, fn, warmup)
    t = event_times(torch, fn, reps)
    flop = 10.0 * w.d * pairs_per_head(w) * w.B * w.Hq
    ms = float(np.median(t))
    tf = flop / (ms * 1e-3) / 1e12
    res = {
        "ms": ms, "ms_p10": float(np.percentile(t, 10)), "ms_p90": float(np.percentile(t, 90)),
        "useful_tflops": tf, "pct_bf16_mfma_peak": 100.0 * tf / MFMA_BF16_PEAK_TFLOPS,
        "useful_flop": flop, "layer_calls": 1,
    }
    del q, k, v, a, dO, lse, o, ws
    return res


def cpu_baseline(w, budget_s=12.0):
    """The oracle (fp64, OpenMP over query rows) on a bounded sample of the
    workload: whole (batch, head) slices, grown until about budget_s of CPU
    work; reported in the headline unit (useful TFLOP/s)."""
    import oracle
    from structured_sparse_causal_amd.inputs import prefill_inputs
    q, k, v, a = prefill_inputs(w)
    per_head_flop = 4.0 * w.d * pairs_per_head(w)
    nthreads = oracle.num_threads()

    def run(nh):
        heads = [(b, h) for b in range(w.B) for h in range(w.Hq)][:nh]
        rows = np.concatenate([(np.int64(b * w.Hq + h) * w.N + np.arange(w.N)) for b, h in heads])
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, a, mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg, rows=rows)
        return time.perf_counter() - t0

    nh, dt = 1, run(1)
    total = w.B * w.Hq
    if dt < budget_s and nh < total:
        nh = int(min(total, max(1, math.floor(budget_s / max(dt, 1e-3)))))
        dt = run(nh)
    flop = per_head_flop * nh
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": "%d of %d (batch, head) slices of %s%s, all %d query rows each, fp64 C oracle; "
                      "%.2f s" % (nh, total, w.name, " (its first application; the other %d apply the same "
                                  "key sets)" % (w.loops - 1) if w.loops > 1 else "", w.N, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="window_loop_bf16")
    ap.add_argument("--no-extras", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, metavar="WORKLOAD",
                    help="time one workload of the hot path and print its statistics only (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU (no sharding or collectives); "
              "--gpus %d is not supported. Run with --gpus 1." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import structured_sparse_causal_amd as sa
    from structured_sparse_causal_amd.inputs import WORKLOADS, prefill_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    sa.load_library()
    dev = torch.device("cuda:0")
    if args.only is not None:
        if args.only == "fused_options":
            print(json.dumps({"workload": args.only, **run_option_workloads(torch, sa, args.steps, args.warmup)}),
                  flush=True)
            return
        if args.only == "decode_layouts":
            print(json.dumps({"workload": args.only,
                              **run_decode_layouts(torch, sa, WORKLOADS["decode_pi_gqa_bf16"], args.steps,
                                                   args.warmup)}), flush=True)
            return
        from structured_sparse_causal_amd.inputs import MASK_WORKLOADS
        if args.only in MASK_WORKLOADS:
            print(json.dumps({"workload": args.only, **run_prefill_workload(torch, sa, MASK_WORKLOADS[args.only],
                                                                           args.steps, args.warmup)}), flush=True)
            return
        if args.only.startswith("bwd_"):
            wx = WORKLOADS[args.only[4:]].replace(loops=1)
            print(json.dumps({"workload": args.only, **run_bwd_workload(torch, sa, wx, args.steps, args.warmup)}),
                  flush=True)
            return
        wx = WORKLOADS[args.only]
        run = run_decode_workload if wx.decode else run_prefill_workload
        print(json.dumps({"workload": wx.name, **run(torch, sa, wx, args.steps, args.warmup)}), flush=True)
        return
    w = WORKLOADS[args.workload]
    if w.decode:
        raise SystemExit("the headline workload must be a prefill workload")
    log("bench: headline %s" % (w,))

    # ---- headline: K timed steps bracketed by synchronisation ---------------
    q, k, v, a = prefill_inputs(w, device=dev)
    prm = dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)
    out = torch.empty_like(q)
    outs = (out, torch.empty_like(q))
    nbytes = sa.fwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, w.mode, w.k_win, w.pi,
                                   w.M, w.seg)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def step():
        if w.loops > 1:
            sa.loop_fwd(q, k, v, a, steps=w.loops, outs=outs, workspace=ws, **prm)
        else:
            sa.fwd(q, k, v, a, out=out, workspace=ws, **prm)

    # Untimed clock settling (at least 0.3 s of steps: the engine clock rises
    # over the first few hundred milliseconds of work), then the W warm-up
    # steps, then the K timed steps.
    settle_t0 = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - settle_t0 < 0.3:
        step()
        settle_steps += 1
        if settle_steps % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    settle_s = time.perf_counter() - settle_t0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    flop, nb = prefill_useful(w)
    flop_step = flop * w.loops
    value = flop_step / (wall / args.steps) / 1e12

    # Dominant kernel: per-launch durations from HIP events on the launch stream.
    # One event pair around K back-to-back steps on the launch stream: the
    # average launch duration as a kernel trace measures it (per-call event
    # pairs add their own gaps to every launch).  Before it, the event pair is
    # exercised once and the kernel runs for ~0.3 s untimed: the first timed
    # event pair of a process and a GPU still raising its clock after an idle
    # host phase both read up to ~15 % slow.
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(st)
    step()
    ev1.record(st)
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.3:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    ev0.record(st)
    for _ in range(args.steps):
        step()
    ev1.record(st)
    torch.cuda.synchronize()
    kern_ms = ev0.elapsed_time(ev1) / args.steps / (w.loops if w.loops > 1 else 1)
    dominant = dominant_kernel(w)
    achieved = flop / (kern_ms * 1e-3) / 1e12
    ai = flop / nb
    bound = "mfma" if ai * HBM_PEAK_GBS / 1000.0 >= MFMA_BF16_PEAK_TFLOPS else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
    else:
        gbs = nb / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": None}
    roof["traffic"] = recorded_traffic(w)
    roof["traffic_over_algorithmic"] = roof["traffic"] / nb if roof["traffic"] is not None else None
    roof["kernel"] = dominant
    roof["kernel_ms"] = kern_ms
    roof["algorithmic_flop_per_launch"] = flop
    roof["algorithmic_bytes_per_launch"] = nb
    log("headline: %.4f ms/step, %.1f useful TFLOP/s (events: %.4f ms/launch)" % (
        ms_step, value, kern_ms))
    # Cold-cache step: a 1 GiB scratch write before each timed step evicts the
    # inputs from L2 and the 256 MB last-level cache, so q, k, v come from HBM.
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(20):
        scratch.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        step()
        e1.record(st)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold_ms = float(np.median(cold))
    cold_tf = flop_step / (cold_ms * 1e-3) / 1e12
    cold_rec = {"ms": cold_ms, "ms_p10": float(np.percentile(cold, 10)), "ms_p90": float(np.percentile(cold, 90)),
                "useful_tflops": cold_tf, "pct_bf16_mfma_peak": 100.0 * cold_tf / MFMA_BF16_PEAK_TFLOPS,
                "steps": len(cold), "warm_over_cold": value / cold_tf,
                "note": "one step after a 1 GiB scratch write (inputs evicted from L2 and the 256 MB "
                        "last-level cache), per-step event pair"}
    log("headline cold-cache: %.4f ms/step" % cold_ms)
    del q, k, v, a, out, outs, ws, scratch
    torch.cuda.empty_cache()

    # ---- the other workloads of the hot path --------------------------------
    extras = {}
    if not args.no_extras:
        for name in ("pi_tiny_f32", "ecp_bf16", "pi_bf16", "window_loop_bf16", "decode_pi_gqa_bf16"):
            wx = WORKLOADS[name]
            log("bench: workload %s" % name)
            reps = 10 if name == "window_loop_bf16" else 30
            if wx.decode:
                extras[name] = run_decode_workload(torch, sa, wx, reps, 3)
            else:
                extras[name] = run_prefill_workload(torch, sa, wx, reps, 3)
            log("  %s" % json.dumps(extras[name]))
            torch.cuda.empty_cache()
        # Further mask modes (forward), at the ECP and looped-window shapes.
        from structured_sparse_causal_amd.inputs import MASK_WORKLOADS
        for name, wx in MASK_WORKLOADS.items():
            log("bench: mask mode %s" % name)
            extras[name] = run_prefill_workload(torch, sa, wx, 10 if wx.d == 128 else 30, 3)
            log("  %s" % json.dumps(extras[name]))
            torch.cuda.empty_cache()
        # Fused gate and epilogue options against the plain calls.
        log("bench: fused options")
        extras["fused_options"] = run_option_workloads(torch, sa, 20, 3)
        log("  %s" % json.dumps(extras["fused_options"]))
        torch.cuda.empty_cache()
        # Serving decode: cache layouts, and throughput over cache lengths.
        wd = WORKLOADS["decode_pi_gqa_bf16"]
        log("bench: decode over paged and ring caches")
        extras["decode_layouts"] = run_decode_layouts(torch, sa, wd, 20, 3)
        log("  %s" % json.dumps(extras["decode_layouts"]))
        torch.cuda.empty_cache()
        flat = {}
        for L in (4096, 8192, 16384, 32768):
            r = run_decode_workload(torch, sa, wd.replace(N=L), 20, 3)
            flat[str(L)] = {k: r[k] for k in ("ms", "tokens_per_s", "useful_GBps", "useful_bytes")}
            torch.cuda.empty_cache()
        extras["decode_cache_length_sweep"] = flat
        log("  decode over cache lengths: %s" % json.dumps(flat))
        # Backward pass (training) of one layer call on the prefill shapes.
        for name in ("ecp_bf16", "pi_bf16", "window_loop_bf16"):
            wx = WORKLOADS[name].replace(loops=1)
            log("bench: backward %s (one layer call)" % name)
            extras["bwd_" + name] = run_bwd_workload(torch, sa, wx, 10 if wx.d == 128 else 30, 3)
            log("  %s" % json.dumps(extras["bwd_" + name]))
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(w)
        log("  %s" % json.dumps(cpu))

    rec = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "k_win": w.k_win, "pi": w.pi, "M": w.M, "seg": w.seg,
                   "loops": w.loops, "parallelism": "none (1 GPU)"},
        "pct_bf16_mfma_peak": 100.0 * value / MFMA_BF16_PEAK_TFLOPS,
        "clock_settle": {"untimed_steps": settle_steps, "seconds": settle_s},
        "roofline": roof,
        "cold_cache": cold_rec,
        "cpu_baseline": cpu,
        "workloads": extras,
        "gpu": torch.cuda.get_device_properties(0).gcnArchName,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
