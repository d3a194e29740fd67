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
