"""Comparison of GPU results with the float64 oracle, for the GPU tests."""
import numpy as np

import oracle
from gpu_device import DeviceProblem, to_device  # noqa: F401

# tolerance on max|gpu - oracle| relative to max|oracle| (fp32 caches / bf16 and fp8 caches)
TOL = {"f32": 1e-5, "bf16": 2e-3, "e4m3fn": 2e-3}


def compare(prob, out, flags, rows=None, tol=None, ref=None):
    """Check GPU output/flags against the oracle; returns (rel err, oracle out, oracle flags)."""
    if ref is None:
        ref_out, ref_flags, _ = oracle.decode_exact(**prob.args(), rows=rows)
    else:
        ref_out, ref_flags = ref
    if rows is not None:
        out, flags = out[rows], flags[rows]
    np.testing.assert_array_equal(flags, ref_flags)
    tol = TOL[prob.kv_dtype] if tol is None else tol
    finite = np.isfinite(ref_out).all(axis=1)
    np.testing.assert_array_equal(np.isnan(out[~finite]), np.isnan(ref_out[~finite]))
    scale = np.abs(ref_out[finite]).max() if finite.any() else 1.0
    err = np.abs(out[finite] - ref_out[finite]).max() if finite.any() else 0.0
    assert err <= tol * scale, "max|err| %.3e > %.1e * max|out| (%.3e)" % (err, tol, scale)
    return err / scale, ref_out, ref_flags
