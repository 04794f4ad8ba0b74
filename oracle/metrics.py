"""Error metric used by every parity check (test infrastructure only).

The contributor guide ("Flash Linear Attention contributor guide", section on
tests) describes ``assert_close`` as: check for NaN first, then report the
error ratio, the RMS of the difference divided by the RMS of the reference.
It is restated here in float64.
"""
import numpy as np
import torch


def _np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def err_ratio(x, ref) -> float:
    """RMS(x - ref) / RMS(ref); raises if x holds NaN or Inf."""
    a, b = _np(x), _np(ref)
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}")
    if not np.isfinite(a).all():
        raise AssertionError("non-finite values in result")
    den = np.sqrt(np.mean(b * b)) if b.size else 0.0
    num = np.sqrt(np.mean((a - b) ** 2)) if a.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)

