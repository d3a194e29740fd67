"""The allocation-free decode entry point (sparse_attn_decode_noalloc) against
the workspace decode (sparse_attn_decode), both through the C ABI: two calls
in a row, the second with a smaller input, each bit-identical to the
workspace call on the same inputs (same kernels, same split plan), and the
first also within the bf16 tolerance of the oracle."""
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


def prm(w):
    return dict(mode=w.mode, k_win=w.k_win, pi=w.pi, M=w.M, seg=w.seg)


def test_noalloc_decode_matches_workspace_decode_twice():
    # 12 and 2 (sequence, KV head) workgroups: far fewer than the compute
    # units, so both calls take the split plan and use the scratch.
    first = Workload("noalloc_pi_gqa", "pi", "bf16", 6, 8, 2, 3000, 128, k_win=300, pi=128, M=6,
                     decode=True, seed=301)
    second = Workload("noalloc_ecp_f32", "ecp", "f32", 2, 4, 2, 500, 64, seg=96, decode=True, seed=302)
    limit = sa.load_library().sparse_attn_decode_noalloc_max_workspace()
    for w in (first, second):
        need = sa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, w.torch_dtype, w.mode, w.k_win, w.pi, w.M,
                                        w.seg)
        assert 0 < need <= limit
        print("noalloc decode %s (partial states %d bytes)" % (w.name, need), flush=True)
        q, kc, vc, lens, a = decode_inputs(w, device=DEV)
        rng = np.random.default_rng(w.seed)
        ragged = torch.from_numpy(rng.integers(1, w.N + 1, w.B).astype(np.int32)).to(DEV)
        for ln in (lens, ragged):
            ref = sa.decode(q, kc, vc, ln, a, **prm(w))
            out = torch.full_like(q, float("nan"))
            got = sa.decode_noalloc(q, kc, vc, ln, a, out=out, **prm(w))
            torch.cuda.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.equal(got, ref), "%s: noalloc decode differs from the workspace decode" % w.name
        if w is first:
            o = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), ragged.cpu(), a.cpu(), **prm(w))
            assert_close(got.float().cpu().numpy(), o, w.dtype, w.name)
        del q, kc, vc, lens, a
