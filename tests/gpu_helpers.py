"""Shared helpers of the GPU parity tests (HIP library vs CPU oracle)."""
import sys

import numpy as np
import torch

# Tolerance for attention outputs against the oracle: max-abs 2e-2 and
# mean-abs 2e-3 (the bf16-compute contract of the hot path), on the error
# divided by max(1, M), where M = sum_j p_j |V_j| / sum_j p_j is the size of
# the terms the output sums (the oracle returns it).  Rounding the weights or
# the output to bf16 (relative 2^-9) moves an output by up to 2^-9 * M, so
# with unit-variance V (M < 1) this is the plain absolute error, and with
# x20 outliers in V (M up to ~80) the bound scales with the data.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(x, dtype=None):
    t = torch.as_tensor(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def assert_close(got, want, what, mag=None, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """got: tensor (any float dtype); want: float64 array of the same shape;
    mag: the oracle's sum_j p_j |V_j| / sum_j p_j for each output (None: |want|)."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    w = np.asarray(want, dtype=np.float64)
    m = np.abs(w) if mag is None else np.asarray(mag, dtype=np.float64)
    assert g.shape == w.shape == m.shape, (what, g.shape, w.shape, m.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    raw = np.abs(g - w)
    err = raw / np.maximum(1.0, m)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    raw_mx = float(raw.max()) if raw.size else 0.0
    print(f"[parity] {what}: max_err={mx:.3e} mean_err={mean:.3e} (raw max-abs {raw_mx:.3e}, "
          f"max M {float(m.max()) if m.size else 0.0:.3g}) n={err.size}", flush=True)
    assert mx <= max_abs, f"{what}: max error {mx:.3e} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean error {mean:.3e} > {mean_abs}"
    return mx, mean
