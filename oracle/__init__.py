"""fp64 CPU oracle for causal structured-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It never imports the
HIP library package and shares no code with it; the heavy loop lives in
``sparse_attn_oracle.c`` (plain C, fp64, OpenMP over query rows) and is loaded
here with ctypes.

The method (one softmax over an explicit key set with an additive log-prior)
is defined on the pages:

* "pi-Attention: Periodic Sparse Transformers for Efficient Long-Context
  Modeling", section 2 items 1-3 -- causal window, periodic skips, gate alpha
  as a log-prior (log alpha on local keys, log(1-alpha) on skip keys).
* "LT2: Linear-Time Looped Transformers", section 2.1 (window-only sparse
  attention) and section 2.2 (looping: the block is applied T times).
* "Efficient Context Propagating Perceiver ...", section 2 (PAR block over a
  pair of consecutive half-segments, causal).
* "Long-context modelling with a hybrid GSS-Transformer" (PHA), methodology
  item 1 (grouped-query attention).

Every function states which of these it follows.  Parity of every function here
is pinned by the ``not gpu`` tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

MODE_PI = 0
MODE_WINDOW = 1
MODE_ECP = 2
MODE_WINDOW_BIDIR = 3
MODE_SSPLIT = 4
MODE_ECP_FULL = 5
MODES = {"pi": MODE_PI, "window": MODE_WINDOW, "ecp": MODE_ECP, "window_bidir": MODE_WINDOW_BIDIR,
         "ssplit": MODE_SSPLIT, "ecp_full": MODE_ECP_FULL}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sparse_attn_oracle.c")
_LIB = os.path.join(_HERE, "libsaoracle.so")
_lock = threading.Lock()
_lib = None

_ERRORS = {-1: "invalid arguments", -2: "alpha missing or outside (0, 1]", -3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                        "-fno-fast-math", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("SA_ORACLE_LIB")   # another build of this oracle (sanitizer runs)
            if not path:
                build(force=False)
                path = _LIB
            lib = ctypes.CDLL(path)
            i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
            lib.orc_key_set.restype = i64
            lib.orc_key_set.argtypes = [i64, i64, i32, i64, i64, i64, i64, vp, vp, i64]
            lib.orc_key_capacity.restype = i64
            lib.orc_key_capacity.argtypes = [i32, i64, i64, i64]
            f64 = ctypes.c_double
            lib.orc_fwd_rows_ex.restype = i32
            lib.orc_fwd_rows_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                            i32, i64, i64, i64, i64, f64, i32, vp, vp, vp, vp, i64,
                                            vp, i64, vp]
            lib.orc_decode_ex.restype = i32
            lib.orc_decode_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          i32, i64, i64, i64, i64, f64, i32, vp, vp, vp, vp, i64, vp]
            lib.orc_lse_rows_ex.restype = i32
            lib.orc_lse_rows_ex.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64,
                                            i32, i64, i64, i64, i64, f64, i32, vp, vp, vp, vp, i64,
                                            vp, i64, vp]
            lib.orc_bwd.restype = i32
            lib.orc_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                    i32, i64, i64, i64, i64, f64, vp, vp, vp, vp]
            lib.orc_num_threads.restype = i32
            lib.orc_set_num_threads.argtypes = [i32]
            _lib = lib
    return _lib


def _mode(mode) -> int:
    if isinstance(mode, str):
        return MODES[mode.lower()]
    return int(mode)


def _f32(x) -> np.ndarray:
    """Widen an input exactly to a contiguous float32 array (bf16 and fp32
    values are exactly representable)."""
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().to("cpu")
        if str(x.dtype) != "torch.float32":
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _check(rc: int):
    if rc != 0:
        raise ValueError("oracle: " + _ERRORS.get(rc, "error %d" % rc))


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


def key_set(i: int, mode, k_win: int = 0, pi: int = 0, M: int = 0, seg: int = 0, N=None):
    """Key set of query position ``i`` of an N-position sequence (default
    N = i + 1, enough for the causal modes) as (positions, labels); label
    0 = local, 1 = skip.  pi-Attention section 2 items 1-2; ECP section 2;
    LT2 section 2.1."""
    lib = _load()
    m = _mode(mode)
    cap = max(1, lib.orc_key_capacity(m, k_win, M, seg))
    keys = np.zeros(cap, dtype=np.int64)
    labels = np.zeros(cap, dtype=np.int32)
    n = lib.orc_key_set(int(i), int(i) + 1 if N is None else int(N), m, int(k_win), int(pi), int(M), int(seg),
                        keys.ctypes.data, labels.ctypes.data, cap)
    if n < 0:
        raise ValueError("oracle: invalid key-set parameters")
    return keys[:n].copy(), labels[:n].copy()


class _Gate:
    """Gate network arguments as the C oracle takes them (fp32 arrays kept
    alive for the call): one linear layer, w [Hq, d] and b [Hq]; or two
    layers with a ReLU hidden layer of width H, w [Hq, H, d], b [Hq, H],
    w2 [Hq, H], b2 [Hq]."""

    def __init__(self, gate_w, gate_b, gate_w2, gate_b2, Hq, d):
        self.arrays = [None, None, None, None]
        self.hidden = 0
        if gate_w is None:
            if gate_b is not None or gate_w2 is not None or gate_b2 is not None:
                raise ValueError("oracle: gate biases or second layer without gate_w")
            return
        w, b = _f32(gate_w), _f32(gate_b)
        if gate_w2 is None:
            if gate_b2 is not None or w.shape != (Hq, d) or b.shape != (Hq,):
                raise ValueError("oracle: linear gate needs gate_w [Hq, d] and gate_b [Hq]")
            self.arrays = [w, b, None, None]
            return
        w2, b2 = _f32(gate_w2), _f32(gate_b2)
        H = w.shape[1] if w.ndim == 3 else -1
        if H < 1 or w.shape != (Hq, H, d) or b.shape != (Hq, H) or w2.shape != (Hq, H) or b2.shape != (Hq,):
            raise ValueError("oracle: gate MLP needs gate_w [Hq, H, d], gate_b [Hq, H], gate_w2 [Hq, H], "
                             "gate_b2 [Hq]")
        self.arrays = [w, b, w2, b2]
        self.hidden = H

    def args(self):
        return [a.ctypes.data if a is not None else None for a in self.arrays] + [self.hidden]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def _out_gate(out, out_gate):
    """Output gate of the LT2 page (section 3): o * sigmoid(g), elementwise."""
    if out_gate is None:
        return out
    g = _f32(out_gate).astype(np.float64)
    return out * _sigmoid(g.reshape(out.shape) if g.size == out.size else g)


def fwd(q, k, v, alpha=None, *, mode, k_win: int = 0, pi: int = 0, M: int = 0,
        seg: int = 0, rows=None, scale=None, cosine: bool = False, gate_w=None, gate_b=None,
        gate_w2=None, gate_b2=None, out_gate=None) -> np.ndarray:
    """Forward attention in fp64.

    q [B,Hq,N,d], k/v [B,Hkv,N,d], alpha [B,Hq,N] (PI only).  With ``rows``
    (flat ids (b*Hq+h)*N+i) returns [len(rows), d]; otherwise [B,Hq,N,d].
    Options: ``scale`` (default 1/sqrt(d)); ``cosine`` scores
    scale * cos(q_i, k_j); the gate network instead of the alpha input:
    ``gate_w`` [Hq,d] / ``gate_b`` [Hq] give alpha = sigmoid(<w_h, q_i> + b_h),
    and with ``gate_w`` [Hq,H,d], ``gate_b`` [Hq,H], ``gate_w2`` [Hq,H],
    ``gate_b2`` [Hq] alpha = sigmoid(sum_u w2_hu relu(<w_hu, q_i> + b_hu) + b2_h);
    ``out_gate`` (shaped like the output): o * sigmoid(out_gate).
    """
    lib = _load()
    q32, k32, v32 = _f32(q), _f32(k), _f32(v)
    B, Hq, N, d = q32.shape
    Hkv = k32.shape[1]
    if k32.shape != (B, Hkv, N, d) or v32.shape != k32.shape:
        raise ValueError("oracle: k/v shape mismatch")
    m = _mode(mode)
    a32 = _f32(alpha) if alpha is not None else None
    if a32 is not None and a32.shape != (B, Hq, N):
        raise ValueError("oracle: alpha shape mismatch")
    if rows is None:
        out = np.empty((B, Hq, N, d), dtype=np.float64)
        sel_p, nsel = None, 0
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
        out = np.empty((sel.size, d), dtype=np.float64)
        sel_p, nsel = sel.ctypes.data, sel.size
    gate = _Gate(gate_w, gate_b, gate_w2, gate_b2, Hq, d)
    rc = lib.orc_fwd_rows_ex(q32.ctypes.data, k32.ctypes.data, v32.ctypes.data,
                             a32.ctypes.data if a32 is not None else None,
                             B, Hq, Hkv, N, d, m, int(k_win), int(pi), int(M), int(seg),
                             1.0 / np.sqrt(d) if scale is None else float(scale), int(bool(cosine)),
                             *gate.args(), sel_p, nsel, out.ctypes.data)
    _check(rc)
    if out_gate is not None and rows is not None:
        out_gate = _f32(out_gate).reshape(-1, d)[np.asarray(rows, dtype=np.int64).ravel()]
    return _out_gate(out, out_gate)


def lse(q, k, alpha=None, *, mode, k_win: int = 0, pi: int = 0, M: int = 0, seg: int = 0,
        rows=None, scale=None, cosine: bool = False, gate_w=None, gate_b=None, gate_w2=None,
        gate_b2=None) -> np.ndarray:
    """Log-sum-exp of each row's scores (natural log), fp64: [B,Hq,N], or
    [len(rows)] for flat row ids."""
    lib = _load()
    q32, k32 = _f32(q), _f32(k)
    B, Hq, N, d = q32.shape
    Hkv = k32.shape[1]
    if k32.shape != (B, Hkv, N, d):
        raise ValueError("oracle: k shape mismatch")
    a32 = _f32(alpha) if alpha is not None else None
    if rows is None:
        out = np.empty((B, Hq, N), dtype=np.float64)
        sel_p, nsel = None, 0
    else:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
        out = np.empty(sel.size, dtype=np.float64)
        sel_p, nsel = sel.ctypes.data, sel.size
    gate = _Gate(gate_w, gate_b, gate_w2, gate_b2, Hq, d)
    rc = lib.orc_lse_rows_ex(q32.ctypes.data, k32.ctypes.data,
                             a32.ctypes.data if a32 is not None else None,
                             B, Hq, Hkv, N, d, _mode(mode), int(k_win), int(pi), int(M), int(seg),
                             1.0 / np.sqrt(d) if scale is None else float(scale), int(bool(cosine)),
                             *gate.args(), sel_p, nsel, out.ctypes.data)
    _check(rc)
    return out


def bwd(q, k, v, alpha, dO, *, mode, k_win: int = 0, pi: int = 0, M: int = 0, seg: int = 0,
        scale=None, out_gate=None):
    """Backward pass in fp64 (the chain rule through the forward definition;
    the gate gradient follows pi-Attention section 2 item 3).
    Returns (dq [B,Hq,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d], dalpha [B,Hq,N] or None).
    With ``out_gate`` g (output y = o * sigmoid(g), LT2 section 3), dO is the
    gradient of y: the attention's output gradient is dO * sigmoid(g), and a
    fifth result dg = dO * o * sigmoid(g) * (1 - sigmoid(g)) is returned."""
    lib = _load()
    q32, k32, v32 = _f32(q), _f32(k), _f32(v)
    do64 = _f32(dO).astype(np.float64)
    dg = None
    if out_gate is not None:
        sg = _sigmoid(_f32(out_gate))
        o = fwd(q, k, v, alpha, mode=mode, k_win=k_win, pi=pi, M=M, seg=seg, scale=scale)
        dg = do64 * o * sg * (1.0 - sg)
        do64 = do64 * sg
    do64 = np.ascontiguousarray(do64)
    B, Hq, N, d = q32.shape
    Hkv = k32.shape[1]
    if k32.shape != (B, Hkv, N, d) or v32.shape != k32.shape or do64.shape != q32.shape:
        raise ValueError("oracle: shape mismatch")
    m = _mode(mode)
    a32 = _f32(alpha) if alpha is not None else None
    dq = np.empty((B, Hq, N, d), dtype=np.float64)
    dk = np.empty((B, Hkv, N, d), dtype=np.float64)
    dv = np.empty((B, Hkv, N, d), dtype=np.float64)
    da = np.zeros((B, Hq, N), dtype=np.float64) if m == MODES["pi"] else None
    rc = lib.orc_bwd(q32.ctypes.data, k32.ctypes.data, v32.ctypes.data,
                     a32.ctypes.data if a32 is not None else None, do64.ctypes.data,
                     B, Hq, Hkv, N, d, m, int(k_win), int(pi), int(M), int(seg),
                     1.0 / np.sqrt(d) if scale is None else float(scale),
                     dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                     da.ctypes.data if da is not None else None)
    _check(rc)
    if dg is not None:
        return dq, dk, dv, da, dg
    return dq, dk, dv, da


def decode(q, k_cache, v_cache, lens, alpha=None, *, mode, k_win: int = 0, pi: int = 0,
           M: int = 0, seg: int = 0, scale=None, cosine: bool = False, gate_w=None, gate_b=None,
           gate_w2=None, gate_b2=None, out_gate=None) -> np.ndarray:
    """Single-token decode in fp64: the query of sequence b is at position
    lens[b]-1 and attends that position's key set inside the cache.
    q [B,Hq,d], caches [B,Hkv,Lmax,d], lens [B], alpha [B,Hq] -> [B,Hq,d]."""
    lib = _load()
    q32, kc, vc = _f32(q), _f32(k_cache), _f32(v_cache)
    B, Hq, d = q32.shape
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    if kc.shape != (B, Hkv, Lmax, d) or vc.shape != kc.shape:
        raise ValueError("oracle: cache shape mismatch")
    if hasattr(lens, "detach"):
        lens = lens.detach().cpu().numpy()
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    a32 = _f32(alpha) if alpha is not None else None
    out = np.empty((B, Hq, d), dtype=np.float64)
    gate = _Gate(gate_w, gate_b, gate_w2, gate_b2, Hq, d)
    rc = lib.orc_decode_ex(q32.ctypes.data, kc.ctypes.data, vc.ctypes.data, ln.ctypes.data,
                           a32.ctypes.data if a32 is not None else None,
                           B, Hq, Hkv, Lmax, d, _mode(mode), int(k_win), int(pi), int(M),
                           int(seg), 1.0 / np.sqrt(d) if scale is None else float(scale),
                           int(bool(cosine)), *gate.args(), out.ctypes.data)
    _check(rc)
    return _out_gate(out, out_gate)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits,
    ties to even), returned as fp64.  Used where an output is stored in bf16
    and read again, as in the looped block below."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                      # x = mant * 2**expo, 0.5 <= |mant| < 1
    quantum = np.maximum(expo - 8, -133)          # bf16 subnormal quantum is 2**-133
    return np.ldexp(np.rint(np.ldexp(x, -quantum)), quantum)


def loop_fwd(q, k, v, alpha=None, *, steps: int, mode, k_win: int = 0, pi: int = 0,
             M: int = 0, seg: int = 0, round_bf16: bool = True):
    """Looped block ("LT2", section 1 and section 2.2): the same attention is
    applied ``steps`` times with Q and K fixed, the output of one application
    becoming the value input of the next.  With ``round_bf16`` every
    intermediate output is rounded to bf16 before it is fed back, as a stored
    bf16 tensor would be.  Returns the list [O_1, ..., O_steps] in fp64."""
    outs = []
    vin = _f32(v)
    for _ in range(steps):
        o = fwd(q, k, vin, alpha, mode=mode, k_win=k_win, pi=pi, M=M, seg=seg)
        outs.append(o)
        vin = (round_to_bf16(o) if round_bf16 else o).astype(np.float32)
    return outs
