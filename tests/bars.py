"""Shared pass/fail bars of the GPU layer tests (host-side numpy only)."""
import numpy as np


def check_y(y, y_codes, y_oracle):
    """max |Y - epilogue(GPU codes)| <= 1e-3 RMS(Y_oracle) over the output,
    and per row <= 1e-3 times that row's RMS of Y_oracle (the BOS-like row
    dominates the overall RMS, so the overall bar alone is loose on the
    ordinary rows)."""
    e = np.abs(np.asarray(y, np.float64) - y_codes)
    yo = np.asarray(y_oracle, np.float64)
    rms = float(np.sqrt(np.mean(yo ** 2)))
    row_rms = np.sqrt(np.mean(yo ** 2, axis=1))
    assert float(e.max()) <= 1e-3 * rms, (float(e.max()), rms)
    bad = e.max(axis=1) > 1e-3 * row_rms
    assert not np.any(bad), (np.nonzero(bad)[0][:8], float(np.max(e.max(axis=1) / row_rms)))
