"""ctypes binding over libsparse_attn.so (C ABI in include/sparse_attn.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  torch supplies device memory (outputs, workspace) and the
current stream.  There is no fallback: if the library is missing or a tensor
is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

MODE_PI = 0
MODE_WINDOW = 1
MODE_ECP = 2
MODE_WINDOW_BIDIR = 3
MODE_SSPLIT = 4
MODE_ECP_FULL = 5
_MODES = {"pi": MODE_PI, "window": MODE_WINDOW, "ecp": MODE_ECP, "window_bidir": MODE_WINDOW_BIDIR,
          "ssplit": MODE_SSPLIT, "ecp_full": MODE_ECP_FULL}

DTYPE_F32 = 0
DTYPE_BF16 = 1
_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_WORKSPACE = 0, -1, -2, -3, -4



class SaOptions(ctypes.Structure):
    """struct sa_options of the C ABI (fused gate and epilogue options)."""
    _fields_ = [("score_scale", ctypes.c_float), ("cosine", ctypes.c_int),
                ("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p), ("out_gate", ctypes.c_void_p),
                ("gate_hidden", ctypes.c_int), ("gate_w2", ctypes.c_void_p), ("gate_b2", ctypes.c_void_p)]


def _gate_hidden(gate_w, gate_b, gate_w2, gate_b2, Hq, d) -> int:
    """Check the gate network's tensors against Hq and d; returns its hidden
    width H (0 for the one-layer gate).  One layer: gate_w [Hq, d], gate_b
    [Hq].  Two layers (ReLU hidden layer): gate_w [Hq, H, d], gate_b [Hq, H],
    gate_w2 [Hq, H], gate_b2 [Hq]."""
    if gate_w is None:
        if gate_b is not None or gate_w2 is not None or gate_b2 is not None:
            raise ValueError("gate biases or second layer given without gate_w")
        return 0
    for t, name in ((gate_w, "gate_w"), (gate_b, "gate_b"), (gate_w2, "gate_w2"), (gate_b2, "gate_b2")):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous fp32 tensor" % name)
    if gate_w2 is None and gate_b2 is None:
        if tuple(gate_w.shape) != (Hq, d) or gate_b is None or tuple(gate_b.shape) != (Hq,):
            raise ValueError("the one-layer gate needs gate_w [Hq, d] and gate_b [Hq]")
        return 0
    H = gate_w.shape[1] if gate_w.dim() == 3 else -1
    if (H < 1 or tuple(gate_w.shape) != (Hq, H, d) or gate_b is None or tuple(gate_b.shape) != (Hq, H)
            or gate_w2 is None or tuple(gate_w2.shape) != (Hq, H) or gate_b2 is None
            or tuple(gate_b2.shape) != (Hq,)):
        raise ValueError("the gate network needs gate_w [Hq, H, d], gate_b [Hq, H], gate_w2 [Hq, H], gate_b2 [Hq]")
    if H > 32:
        raise ValueError("the gate network's hidden width must be at most 32")
    return H


def _options(score_scale=0.0, cosine=False, gate_w=None, gate_b=None, out_gate=None, gate_w2=None,
             gate_b2=None, gate_hidden=0):
    """SaOptions for the given keywords, or None when all are off."""
    if (not score_scale and not cosine and gate_w is None and gate_b is None and out_gate is None
            and gate_w2 is None and gate_b2 is None):
        return None
    for t, name in ((gate_w, "gate_w"), (gate_b, "gate_b"), (gate_w2, "gate_w2"), (gate_b2, "gate_b2")):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("%s must be fp32" % name)
    return SaOptions(float(score_scale), int(bool(cosine)),
                     None if gate_w is None else gate_w.data_ptr(),
                     None if gate_b is None else gate_b.data_ptr(),
                     None if out_gate is None else out_gate.data_ptr(),
                     int(gate_hidden),
                     None if gate_w2 is None else gate_w2.data_ptr(),
                     None if gate_b2 is None else gate_b2.data_ptr())


_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")
_lock = threading.Lock()
_lib = None

EXPORTED = ("sparse_attn_fwd_workspace_size", "sparse_attn_fwd", "sparse_attn_fwd_lse",
            "sparse_attn_bwd_workspace_size", "sparse_attn_bwd",
            "sparse_attn_decode_workspace_size", "sparse_attn_decode",
            "sparse_attn_decode_ring_workspace_size", "sparse_attn_decode_ring",
            "sparse_attn_decode_paged_workspace_size", "sparse_attn_decode_paged",
            "sparse_attn_fwd_ex_workspace_size", "sparse_attn_fwd_ex", "sparse_attn_decode_ex",
            "sparse_attn_bwd_ex_workspace_size", "sparse_attn_bwd_ex",
            "sparse_attn_decode_noalloc_max_workspace", "sparse_attn_decode_noalloc",
            "sparse_attn_status_string", "sparse_attn_last_error", "sparse_attn_version")


class SparseAttnError(RuntimeError):
    """A launch or HIP failure reported by the library."""


def library_path() -> str:
    """The library this binding loads: libsparse_attn.so beside this file, or
    the build named by the SPARSE_ATTN_LIB environment variable (another
    build of the same sources, e.g. one with host-side sanitizers)."""
    return os.environ.get("SPARSE_ATTN_LIB") or _LIB_PATH


def load_library():
    """Load libsparse_attn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("libsparse_attn.so is not built (%s); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
        lib = ctypes.CDLL(path)
        i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        lib.sparse_attn_fwd_workspace_size.restype = sz
        lib.sparse_attn_fwd_workspace_size.argtypes = [i] * 11
        lib.sparse_attn_fwd.restype = i
        lib.sparse_attn_fwd.argtypes = [vp] * 5 + [i] * 11 + [vp, sz, vp]
        lib.sparse_attn_fwd_lse.restype = i
        lib.sparse_attn_fwd_lse.argtypes = [vp] * 6 + [i] * 11 + [vp, sz, vp]
        lib.sparse_attn_bwd_workspace_size.restype = sz
        lib.sparse_attn_bwd_workspace_size.argtypes = [i] * 11
        lib.sparse_attn_bwd.restype = i
        lib.sparse_attn_bwd.argtypes = [vp] * 11 + [i] * 11 + [vp, sz, vp]
        lib.sparse_attn_decode_ring_workspace_size.restype = sz
        lib.sparse_attn_decode_ring_workspace_size.argtypes = [i] * 11
        lib.sparse_attn_decode_ring.restype = i
        lib.sparse_attn_decode_ring.argtypes = [vp] * 6 + [i] * 11 + [vp, sz, vp]
        lib.sparse_attn_decode_paged_workspace_size.restype = sz
        lib.sparse_attn_decode_paged_workspace_size.argtypes = [i] * 12
        lib.sparse_attn_decode_paged.restype = i
        lib.sparse_attn_decode_paged.argtypes = [vp] * 7 + [i] * 13 + [vp, sz, vp]
        op = ctypes.POINTER(SaOptions)
        lib.sparse_attn_fwd_ex_workspace_size.restype = sz
        lib.sparse_attn_fwd_ex_workspace_size.argtypes = [i] * 11 + [op]
        lib.sparse_attn_fwd_ex.restype = i
        lib.sparse_attn_fwd_ex.argtypes = [vp] * 6 + [i] * 11 + [op, vp, sz, vp]
        lib.sparse_attn_decode_ex.restype = i
        lib.sparse_attn_decode_ex.argtypes = [vp] * 6 + [i] * 11 + [op, vp, sz, vp]
        lib.sparse_attn_bwd_ex_workspace_size.restype = sz
        lib.sparse_attn_bwd_ex_workspace_size.argtypes = [i] * 11 + [op]
        lib.sparse_attn_bwd_ex.restype = i
        lib.sparse_attn_bwd_ex.argtypes = [vp] * 11 + [i] * 11 + [op, vp, vp, sz, vp]
        lib.sparse_attn_decode_workspace_size.restype = sz
        lib.sparse_attn_decode_workspace_size.argtypes = [i] * 11
        lib.sparse_attn_decode.restype = i
        lib.sparse_attn_decode.argtypes = [vp] * 6 + [i] * 11 + [vp, sz, vp]
        lib.sparse_attn_decode_noalloc_max_workspace.restype = sz
        lib.sparse_attn_decode_noalloc_max_workspace.argtypes = []
        lib.sparse_attn_decode_noalloc.restype = i
        lib.sparse_attn_decode_noalloc.argtypes = [vp] * 6 + [i] * 11 + [vp]
        lib.sparse_attn_status_string.restype = ctypes.c_char_p
        lib.sparse_attn_status_string.argtypes = [i]
        lib.sparse_attn_last_error.restype = ctypes.c_char_p
        lib.sparse_attn_last_error.argtypes = []
        lib.sparse_attn_version.restype = i
        lib.sparse_attn_version.argtypes = []
        _lib = lib
        return lib


def _raise(lib, rc: int, what: str):
    detail = lib.sparse_attn_last_error().decode()
    msg = "%s: %s (%s)" % (what, lib.sparse_attn_status_string(rc).decode(), detail)
    if rc in (SA_ERR_INVALID, SA_ERR_WORKSPACE):
        raise ValueError(msg)
    if rc == SA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SparseAttnError(msg)


def _mode(mode) -> int:
    if isinstance(mode, str):
        return _MODES[mode.lower()]
    return int(mode)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (got %s)" % t.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd_workspace_size(B, Hq, Hkv, N, d, dtype, mode, k_win=0, pi=0, M=0, seg=0) -> int:
    lib = load_library()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.sparse_attn_fwd_workspace_size(B, Hq, Hkv, N, d, dt, _mode(mode),
                                                  k_win, pi, M, seg))


def decode_workspace_size(B, Hq, Hkv, Lmax, d, dtype, mode, k_win=0, pi=0, M=0, seg=0) -> int:
    lib = load_library()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.sparse_attn_decode_workspace_size(B, Hq, Hkv, Lmax, d, dt, _mode(mode),
                                                     k_win, pi, M, seg))


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return workspace
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def fwd(q, k, v, alpha=None, *, mode, k_win: int = 0, pi: int = 0, M: int = 0, seg: int = 0,
        out=None, workspace=None, lse=None, score_scale: float = 0.0, cosine: bool = False,
        gate_w=None, gate_b=None, out_gate=None, gate_w2=None, gate_b2=None):
    """Prefill forward: q [B,Hq,N,d], k/v [B,Hkv,N,d] (bf16 or fp32, on the
    GPU), alpha [B,Hq,N] fp32 for the gated mode.  Returns o [B,Hq,N,d].
    With ``lse`` (an fp32 [B,Hq,N] tensor) the row log-sum-exp is written
    too (the training forward).  Options (sa_options): score_scale, cosine,
    the gate network on the query in place of alpha (gate_w [Hq,d] / gate_b
    [Hq]: one layer; gate_w [Hq,H,d] / gate_b [Hq,H] / gate_w2 [Hq,H] /
    gate_b2 [Hq]: two layers, ReLU hidden layer), out_gate (like o)."""
    lib = load_library()
    _need_gpu(q, k, v, alpha, out, workspace, gate_w, gate_b, out_gate, gate_w2, gate_b2)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-d [B, H, N, d]")
    hid = _gate_hidden(gate_w, gate_b, gate_w2, gate_b2, q.shape[1], q.shape[3])
    opt = _options(score_scale, cosine, gate_w, gate_b, out_gate, gate_w2, gate_b2, hid)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise NotImplementedError("q, k, v must share dtype bf16 or fp32")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k/v shape %s/%s does not match q %s" % (tuple(k.shape), tuple(v.shape),
                                                                 tuple(q.shape)))
    m = _mode(mode)
    if alpha is not None:
        if alpha.dtype != torch.float32 or tuple(alpha.shape) != (B, Hq, N):
            raise ValueError("alpha must be fp32 [B, Hq, N]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    dt = _DTYPES[q.dtype]
    if opt is not None:
        if out_gate is not None and (out_gate.shape != q.shape or out_gate.dtype != q.dtype):
            raise ValueError("out_gate must match o")
        if lse is not None:
            _need_gpu(lse)
            if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
                raise ValueError("lse must be fp32 [B, Hq, N]")
        nbytes = int(lib.sparse_attn_fwd_ex_workspace_size(B, Hq, Hkv, N, d, dt, m, k_win, pi, M, seg,
                                                           ctypes.byref(opt)))
        ws = _workspace(nbytes, q.device, workspace)
        rc = lib.sparse_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(out), _ptr(lse),
                                    B, Hq, Hkv, N, d, dt, m, int(k_win), int(pi), int(M), int(seg),
                                    ctypes.byref(opt), _ptr(ws), nbytes if ws is not None else 0,
                                    _stream(q.device))
        if rc != SA_OK:
            _raise(lib, rc, "sparse_attn_fwd_ex")
        return out
    nbytes = int(lib.sparse_attn_fwd_workspace_size(B, Hq, Hkv, N, d, dt, m, k_win, pi, M, seg))
    ws = _workspace(nbytes, q.device, workspace)
    if lse is None:
        rc = lib.sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(out),
                                 B, Hq, Hkv, N, d, dt, m, int(k_win), int(pi), int(M), int(seg),
                                 _ptr(ws), nbytes if ws is not None else 0, _stream(q.device))
    else:
        _need_gpu(lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous fp32 [B, Hq, N] tensor")
        rc = lib.sparse_attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(out), _ptr(lse),
                                     B, Hq, Hkv, N, d, dt, m, int(k_win), int(pi), int(M), int(seg),
                                     _ptr(ws), nbytes if ws is not None else 0, _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_fwd")
    return out


def bwd_workspace_size(B, Hq, Hkv, N, d, dtype, mode, k_win=0, pi=0, M=0, seg=0) -> int:
    lib = load_library()
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib.sparse_attn_bwd_workspace_size(B, Hq, Hkv, N, d, dt, _mode(mode), k_win, pi, M, seg))


def bwd(q, k, v, alpha, o, lse, dO, *, mode, k_win: int = 0, pi: int = 0, M: int = 0,
        seg: int = 0, workspace=None, score_scale: float = 0.0, out_gate=None):
    """Backward pass (bf16): gradients given dO for the forward that produced
    o and lse (``fwd(..., lse=...)``).  Returns (dq, dk, dv, dalpha); dalpha
    is an fp32 [B,Hq,N] tensor for the gated mode with alpha, else None.
    With ``out_gate`` (o is then the gated output) a fifth result dgate."""
    lib = load_library()
    _need_gpu(q, k, v, alpha, o, lse, dO, workspace, out_gate)
    opt = _options(score_scale, False, None, None, out_gate)
    if q.dtype != torch.bfloat16 or any(t.dtype != torch.bfloat16 for t in (k, v, o, dO)):
        raise NotImplementedError("the backward pass takes bf16 q, k, v, o, dO")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, d) or v.shape != k.shape or o.shape != q.shape or dO.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dO")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be fp32 [B, Hq, N]")
    m = _mode(mode)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dalpha = torch.empty_like(alpha) if (alpha is not None and m == MODE_PI) else None
    if opt is not None:
        dgate = torch.empty_like(o) if out_gate is not None else None
        nbytes = int(lib.sparse_attn_bwd_ex_workspace_size(B, Hq, Hkv, N, d, DTYPE_BF16, m, k_win, pi, M, seg,
                                                           ctypes.byref(opt)))
        ws = _workspace(nbytes, q.device, workspace)
        rc = lib.sparse_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse), _ptr(dO),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha),
                                    B, Hq, Hkv, N, d, DTYPE_BF16, m, int(k_win), int(pi), int(M), int(seg),
                                    ctypes.byref(opt), _ptr(dgate), _ptr(ws), nbytes, _stream(q.device))
        if rc != SA_OK:
            _raise(lib, rc, "sparse_attn_bwd_ex")
        return (dq, dk, dv, dalpha, dgate) if out_gate is not None else (dq, dk, dv, dalpha)
    nbytes = int(lib.sparse_attn_bwd_workspace_size(B, Hq, Hkv, N, d, DTYPE_BF16, m, k_win, pi, M, seg))
    ws = _workspace(nbytes, q.device, workspace)
    rc = lib.sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse), _ptr(dO),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha),
                             B, Hq, Hkv, N, d, DTYPE_BF16, m, int(k_win), int(pi), int(M), int(seg),
                             _ptr(ws), nbytes, _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_bwd")
    return dq, dk, dv, dalpha


class _Attention(torch.autograd.Function):
    """torch autograd over the library: the training forward (o and the row
    log-sum-exp, sparse_attn_fwd_lse / _ex) and sparse_attn_bwd(_ex) for the
    gradients.  No arithmetic here: both directions run in the HIP kernels."""

    @staticmethod
    def forward(ctx, q, k, v, alpha, out_gate, prm):
        B, Hq, N, _ = q.shape
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        o = fwd(q, k, v, alpha, lse=lse, out_gate=out_gate, **prm)
        ctx.prm = prm
        ctx.save_for_backward(q, k, v, alpha, out_gate, o, lse)
        return o

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, dO):
        q, k, v, alpha, out_gate, o, lse = ctx.saved_tensors
        r = bwd(q, k, v, alpha, o, lse, dO.contiguous(), out_gate=out_gate, **ctx.prm)
        dalpha = r[3] if ctx.needs_input_grad[3] else None
        dgate = r[4] if out_gate is not None and ctx.needs_input_grad[4] else None
        return r[0], r[1], r[2], dalpha, dgate, None


def attention(q, k, v, alpha=None, *, mode, k_win: int = 0, pi: int = 0, M: int = 0, seg: int = 0,
              score_scale: float = 0.0, out_gate=None):
    """Differentiable prefill attention for training (torch autograd; bf16
    q, k, v [B,H,N,d], contiguous, on the GPU): the forward keeps o and the
    row log-sum-exp, the backward returns dq, dk, dv, dalpha (PI mode with
    alpha) and d(out_gate).  Cosine scores or a gate network compose in the
    caller: normalise q, k and pass the scale, or form alpha, and autograd
    carries the gradients through them."""
    prm = dict(mode=mode, k_win=int(k_win), pi=int(pi), M=int(M), seg=int(seg), score_scale=float(score_scale))
    return _Attention.apply(q, k, v, alpha, out_gate, prm)


def decode(q, k_cache, v_cache, cache_lens, alpha=None, *, mode, k_win: int = 0, pi: int = 0,
           M: int = 0, seg: int = 0, out=None, workspace=None, score_scale: float = 0.0,
           cosine: bool = False, gate_w=None, gate_b=None, out_gate=None, gate_w2=None, gate_b2=None):
    """Single-token decode: q [B,Hq,d], caches [B,Hkv,Lmax,d], cache_lens [B]
    int32 on the GPU, alpha [B,Hq] fp32 for the gated mode.  Returns o [B,Hq,d].
    Options as for ``fwd`` (bf16 only); out_gate is [B,Hq,d]."""
    lib = load_library()
    _need_gpu(q, k_cache, v_cache, cache_lens, alpha, out, workspace, gate_w, gate_b, out_gate, gate_w2, gate_b2)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and caches [B, Hkv, Lmax, d]")
    hid = _gate_hidden(gate_w, gate_b, gate_w2, gate_b2, q.shape[1], q.shape[2])
    opt = _options(score_scale, cosine, gate_w, gate_b, out_gate, gate_w2, gate_b2, hid)
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise NotImplementedError("q and caches must share dtype bf16 or fp32")
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Lmax, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    if alpha is not None and (alpha.dtype != torch.float32 or tuple(alpha.shape) != (B, Hq)):
        raise ValueError("alpha must be fp32 [B, Hq]")
    m = _mode(mode)
    if out is None:
        out = torch.empty_like(q)
    dt = _DTYPES[q.dtype]
    nbytes = int(lib.sparse_attn_decode_workspace_size(B, Hq, Hkv, Lmax, d, dt, m, k_win, pi,
                                                       M, seg))
    ws = _workspace(nbytes, q.device, workspace)
    if opt is not None:
        if out_gate is not None and (out_gate.shape != q.shape or out_gate.dtype != q.dtype):
            raise ValueError("out_gate must match o")
        rc = lib.sparse_attn_decode_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens),
                                       _ptr(alpha), _ptr(out), B, Hq, Hkv, Lmax, d, dt, m,
                                       int(k_win), int(pi), int(M), int(seg), ctypes.byref(opt), _ptr(ws),
                                       nbytes if ws is not None else 0, _stream(q.device))
        if rc != SA_OK:
            _raise(lib, rc, "sparse_attn_decode_ex")
        return out
    rc = lib.sparse_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens),
                                _ptr(alpha), _ptr(out), B, Hq, Hkv, Lmax, d, dt, m,
                                int(k_win), int(pi), int(M), int(seg), _ptr(ws),
                                nbytes if ws is not None else 0, _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, cache_lens, alpha=None, *, mode, k_win: int = 0, pi: int = 0,
                   M: int = 0, seg: int = 0, out=None):
    """The decode of ``decode`` through the allocation-free entry point: no
    workspace (the library's per-GPU device scratch holds the partial
    states).  With ``out`` given, this call allocates nothing either."""
    lib = load_library()
    _need_gpu(q, k_cache, v_cache, cache_lens, alpha, out)
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and caches [B, Hkv, Lmax, d]")
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise NotImplementedError("q and caches must share dtype bf16 or fp32")
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Lmax, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    if alpha is not None and (alpha.dtype != torch.float32 or tuple(alpha.shape) != (B, Hq)):
        raise ValueError("alpha must be fp32 [B, Hq]")
    if out is None:
        out = torch.empty_like(q)
    rc = lib.sparse_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens),
                                        _ptr(alpha), _ptr(out), B, Hq, Hkv, Lmax, d, _DTYPES[q.dtype],
                                        _mode(mode), int(k_win), int(pi), int(M), int(seg), _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_decode_noalloc")
    return out


def loop_fwd(q, k, v, alpha=None, *, steps: int, mode, k_win: int = 0, pi: int = 0, M: int = 0,
             seg: int = 0, outs=None, workspace=None):
    """Looped block: apply the attention ``steps`` times with q, k fixed, the
    output of one application becoming the value input of the next ("LT2",
    section 1 and section 2.2).  Two ping-pong output buffers are used (an
    output never aliases its own value input).  Returns the last output."""
    if outs is None:
        outs = (torch.empty_like(q), torch.empty_like(q) if steps > 1 else None)
    vin = v
    o = None
    for t in range(steps):
        o = fwd(q, k, vin, alpha, mode=mode, k_win=k_win, pi=pi, M=M, seg=seg,
                out=outs[t % 2], workspace=workspace)
        vin = o
    return o


def decode_ring(q, k_ring, v_ring, cache_lens, alpha=None, *, mode, k_win: int = 0, pi: int = 0,
                M: int = 0, seg: int = 0, out=None, workspace=None):
    """Decode over ring caches [B,Hkv,R,d] (position p in slot p mod R); bf16.
    cache_lens [B] int32 on the GPU counts the tokens written (query at len-1)."""
    lib = load_library()
    _need_gpu(q, k_ring, v_ring, cache_lens, alpha, out, workspace)
    if q.dim() != 3 or k_ring.dim() != 4 or v_ring.shape != k_ring.shape:
        raise ValueError("q must be [B, Hq, d] and rings [B, Hkv, R, d]")
    if q.dtype != torch.bfloat16 or k_ring.dtype != q.dtype or v_ring.dtype != q.dtype:
        raise NotImplementedError("ring caches take bf16 q and caches")
    B, Hq, d = q.shape
    Hkv, R = k_ring.shape[1], k_ring.shape[2]
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    m = _mode(mode)
    out = torch.empty_like(q) if out is None else out
    nbytes = int(lib.sparse_attn_decode_ring_workspace_size(B, Hq, Hkv, R, d, DTYPE_BF16, m, k_win, pi, M, seg))
    ws = _workspace(max(nbytes, 256), q.device, workspace)
    rc = lib.sparse_attn_decode_ring(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(cache_lens), _ptr(alpha), _ptr(out),
                                     B, Hq, Hkv, R, d, DTYPE_BF16, m, int(k_win), int(pi), int(M), int(seg),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_decode_ring")
    return out


def decode_paged(q, k_pages, v_pages, block_table, cache_lens, alpha=None, *, mode, k_win: int = 0,
                 pi: int = 0, M: int = 0, seg: int = 0, out=None, workspace=None):
    """Decode over paged caches: pools [num_pages,Hkv,page_size,d], block_table
    [B,max_pages] int32 (physical page of each logical page); bf16."""
    lib = load_library()
    _need_gpu(q, k_pages, v_pages, block_table, cache_lens, alpha, out, workspace)
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape or block_table.dim() != 2:
        raise ValueError("q [B, Hq, d], pages [num_pages, Hkv, page_size, d], block_table [B, max_pages]")
    if q.dtype != torch.bfloat16 or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise NotImplementedError("paged caches take bf16 q and caches")
    B, Hq, d = q.shape
    num_pages, Hkv, P = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if block_table.dtype != torch.int32 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    max_pages = block_table.shape[1]
    m = _mode(mode)
    out = torch.empty_like(q) if out is None else out
    nbytes = int(lib.sparse_attn_decode_paged_workspace_size(B, Hq, Hkv, P, max_pages, d, DTYPE_BF16, m, k_win,
                                                              pi, M, seg))
    ws = _workspace(max(nbytes, 256), q.device, workspace)
    rc = lib.sparse_attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(cache_lens),
                                      _ptr(alpha), _ptr(out), B, Hq, Hkv, num_pages, P, max_pages, d, DTYPE_BF16, m,
                                      int(k_win), int(pi), int(M), int(seg), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(q.device))
    if rc != SA_OK:
        _raise(lib, rc, "sparse_attn_decode_paged")
    return out
