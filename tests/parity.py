"""Comparison gates shared by the parity tests.

Tolerances of the hot path, stated for the outputs against the fp64 oracle on
identical input bits:

* bf16 I/O: max |diff| <= 2e-2 and mean |diff| <= 2e-3 (absolute), plus two
  relative gates, because several workloads have outputs of rms ~3e-3 where an
  all-zero output would nearly pass the absolute bounds:
  mean|diff| / mean|ref| <= 1e-2 and max|diff| / max|ref| <= 2e-2.
* fp32 I/O: max |diff| <= 1e-5.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_MEAN_REL = 1e-2
BF16_MAX_REL = 2e-2
F32_MAX_ABS = 1e-5


def error_stats(out, ref) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise AssertionError("shape mismatch %s vs %s" % (out.shape, ref.shape))
    diff = np.abs(out - ref)
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "mean_abs": float(diff.mean()) if diff.size else 0.0,
        "mean_ref": float(np.abs(ref).mean()) if ref.size else 0.0,
        "max_ref": float(np.abs(ref).max()) if ref.size else 0.0,
        "finite": bool(np.isfinite(out).all()),
    }


def gate_failures(out, ref, dtype: str) -> list:
    """List of violated gates (empty when the output passes)."""
    s = error_stats(out, ref)
    bad = []
    if not s["finite"]:
        bad.append("non-finite output")
    if dtype == "f32":
        if s["max_abs"] > F32_MAX_ABS:
            bad.append("max_abs %.3e > %.1e" % (s["max_abs"], F32_MAX_ABS))
        return bad
    if s["max_abs"] > BF16_MAX_ABS:
        bad.append("max_abs %.3e > %.1e" % (s["max_abs"], BF16_MAX_ABS))
    if s["mean_abs"] > BF16_MEAN_ABS:
        bad.append("mean_abs %.3e > %.1e" % (s["mean_abs"], BF16_MEAN_ABS))
    if s["mean_ref"] > 0 and s["mean_abs"] / s["mean_ref"] > BF16_MEAN_REL:
        bad.append("mean_rel %.3e > %.1e" % (s["mean_abs"] / s["mean_ref"], BF16_MEAN_REL))
    if s["max_ref"] > 0 and s["max_abs"] / s["max_ref"] > BF16_MAX_REL:
        bad.append("max_rel %.3e > %.1e" % (s["max_abs"] / s["max_ref"], BF16_MAX_REL))
    return bad


def assert_close(out, ref, dtype: str, what: str = ""):
    bad = gate_failures(out, ref, dtype)
    if bad:
        s = error_stats(out, ref)
        raise AssertionError("%s: %s (stats %s)" % (what, "; ".join(bad), s))


# Gradients of the bf16 backward pass against the fp64 oracle.  The kernels
# round P and dS to bf16 (unit roundoff 2^-9 = 2e-3) before the MFMA products
# and take D_i = dO_i . o_i from the bf16 forward output, so each gradient
# entry carries a relative error of a few 2^-9 on terms of mixed sign; the
# gates are relative to the gradient's own scale (gradients have no natural
# absolute scale): mean|diff| <= 1.5e-2 * mean|ref|, max|diff| <= 3e-2 * max|ref|.
GRAD_MEAN_REL = 1.5e-2
GRAD_MAX_REL = 3e-2


def grad_failures(out, ref) -> list:
    s = error_stats(out, ref)
    bad = []
    if not s["finite"]:
        bad.append("non-finite gradient")
    if s["mean_abs"] > GRAD_MEAN_REL * s["mean_ref"] + 1e-6:
        bad.append("mean_rel %.3e > %.1e" % (s["mean_abs"] / max(s["mean_ref"], 1e-30), GRAD_MEAN_REL))
    if s["max_abs"] > GRAD_MAX_REL * s["max_ref"] + 1e-6:
        bad.append("max_rel %.3e > %.1e" % (s["max_abs"] / max(s["max_ref"], 1e-30), GRAD_MAX_REL))
    return bad


def assert_grad_close(out, ref, what: str = ""):
    bad = grad_failures(out, ref)
    s = error_stats(out, ref)
    print("%s: max_abs %.3e (max_ref %.3e) mean_abs %.3e (mean_ref %.3e)" % (
        what, s["max_abs"], s["max_ref"], s["mean_abs"], s["mean_ref"]), flush=True)
    if bad:
        raise AssertionError("%s: %s (stats %s)" % (what, "; ".join(bad), s))
