"""Seeded synthetic inputs and the workload table.

This module only draws random numbers and casts them; it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle are fed from it, so
both see identical input bits.

Recipe (fixed order of draws from one ``torch.Generator`` seeded per workload):
q, k, v ~ N(0, 1) in fp32 (optionally divided by sqrt(d)), cast to the I/O
dtype with round-to-nearest-even, then alpha = sigmoid(N(0, 1)) kept in fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the hot path."""
    name: str
    mode: str            # "pi" | "window" | "ecp"
    dtype: str           # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int               # sequence length (prefill) or cache length (decode)
    d: int
    k_win: int = 0
    pi: int = 0
    M: int = 0
    seg: int = 0
    scale_inputs: bool = False   # divide q, k, v by sqrt(d) after drawing
    loops: int = 1               # looped block: output fed back as the next V
    decode: bool = False
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the hot path (seed = index + 1).
WORKLOADS = {
    "pi_tiny_f32": Workload("pi_tiny_f32", "pi", "f32", 1, 2, 2, 256, 64,
                            k_win=32, pi=64, M=3, seed=1),
    "ecp_bf16": Workload("ecp_bf16", "ecp", "bf16", 4, 12, 12, 4096, 64,
                         seg=512, scale_inputs=True, seed=2),
    "pi_bf16": Workload("pi_bf16", "pi", "bf16", 2, 16, 16, 16384, 64,
                        k_win=256, pi=1024, M=15, seed=3),
    "window_loop_bf16": Workload("window_loop_bf16", "window", "bf16", 1, 32, 32, 65536, 128,
                                 k_win=1024, scale_inputs=True, loops=4, seed=4),
    "decode_pi_gqa_bf16": Workload("decode_pi_gqa_bf16", "pi", "bf16", 64, 32, 8, 32768, 128,
                                   k_win=2048, pi=2048, M=15, decode=True, seed=5),
}


# The further mask modes at the workload scales above (forward measured in the
# benchmark; seeds continue the numbering).
MASK_WORKLOADS = {
    "window_bidir_bf16": Workload("window_bidir_bf16", "window_bidir", "bf16", 1, 32, 32, 65536, 128,
                                  k_win=1024, scale_inputs=True, seed=6),
    "ssplit_bf16": Workload("ssplit_bf16", "ssplit", "bf16", 4, 12, 12, 4096, 64, seg=512,
                            scale_inputs=True, seed=7),
    "ecp_full_bf16": Workload("ecp_full_bf16", "ecp_full", "bf16", 4, 12, 12, 4096, 64, seg=512,
                              scale_inputs=True, seed=8),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, gen, device, scale: Optional[float]) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale is not None:
        x.mul_(scale)
    return x


def prefill_inputs(w: Workload, device="cpu", seed: Optional[int] = None):
    """q [B,Hq,N,d], k, v [B,Hkv,N,d] in the workload's dtype; alpha [B,Hq,N]
    fp32 for the gated mode (None otherwise)."""
    dev = torch.device(device)
    gen = _gen(w.seed if seed is None else seed, dev)
    sc = 1.0 / math.sqrt(w.d) if w.scale_inputs else None
    q = _normal((w.B, w.Hq, w.N, w.d), gen, dev, sc).to(w.torch_dtype)
    k = _normal((w.B, w.Hkv, w.N, w.d), gen, dev, sc).to(w.torch_dtype)
    v = _normal((w.B, w.Hkv, w.N, w.d), gen, dev, sc).to(w.torch_dtype)
    alpha = None
    if w.mode == "pi":
        alpha = torch.sigmoid(_normal((w.B, w.Hq, w.N), gen, dev, None))
    return q, k, v, alpha


def decode_inputs(w: Workload, device="cpu", seed: Optional[int] = None, chunk_rows: int = 1 << 22):
    """q [B,Hq,d], k_cache, v_cache [B,Hkv,L,d] in the workload's dtype,
    lens [B] int32 (every cache full: lens = L), alpha [B,Hq] fp32 (gated mode).

    The caches are drawn in fixed chunks of rows so host memory stays bounded;
    the chunking is part of the recipe (same seed, same bits)."""
    dev = torch.device(device)
    gen = _gen(w.seed if seed is None else seed, dev)
    sc = 1.0 / math.sqrt(w.d) if w.scale_inputs else None
    q = _normal((w.B, w.Hq, w.d), gen, dev, sc).to(w.torch_dtype)
    caches = []
    for _ in range(2):
        c = torch.empty((w.B * w.Hkv * w.N, w.d), dtype=w.torch_dtype, device=dev)
        for r0 in range(0, c.shape[0], chunk_rows):
            r1 = min(c.shape[0], r0 + chunk_rows)
            c[r0:r1] = _normal((r1 - r0, w.d), gen, dev, sc).to(w.torch_dtype)
        caches.append(c.view(w.B, w.Hkv, w.N, w.d))
    lens = torch.full((w.B,), w.N, dtype=torch.int32, device=dev)
    alpha = None
    if w.mode == "pi":
        alpha = torch.sigmoid(_normal((w.B, w.Hq), gen, dev, None))
    return q, caches[0], caches[1], lens, alpha


def grad_output(w: Workload, device="cpu", seed: Optional[int] = None):
    """dO [B,Hq,N,d] ~ N(0, 1) in the workload's dtype, from its own generator
    (seed + 7919) so the forward inputs keep their bits."""
    dev = torch.device(device)
    gen = _gen((w.seed if seed is None else seed) + 7919, dev)
    return _normal((w.B, w.Hq, w.N, w.d), gen, dev, None).to(w.torch_dtype)
