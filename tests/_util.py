"""Helpers shared by the tests (comparison metric, tensor conversion)."""
import numpy as np
import torch

# Tolerances on the floored relative error below: 1e-4 for fp32 inputs and 2e-2
# for bf16 and fp16 inputs with fp32 state (both 16-bit types reach the matrix
# products as bf16, whose rounding dominates the error).
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 2e-2}


def f64(t):
    """Exact float64 copy (numpy) of a tensor of any floating dtype."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(x, y):
    """max_i |x_i - y_i| / max(|y_i|, rms(y)), y the oracle.

    A plain elementwise ratio is meaningless where the oracle value is near
    zero, so the scale is floored at the tensor's RMS.  An all-zero reference
    compares absolute values."""
    x, y = f64(x), f64(y)
    assert x.shape == y.shape, (x.shape, y.shape)
    if y.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(y * y)))
    if rms == 0.0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - y) / np.maximum(np.abs(y), rms)))


def assert_close(x, y, tol, what=""):
    e = rel_err(x, y)
    assert np.all(np.isfinite(f64(x))), "%s: non-finite values" % what
    assert e <= tol, "%s: floored relative error %.3e > %.1e" % (what, e, tol)
    return e
