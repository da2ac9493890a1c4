"""Shared helpers of the GPU parity tests (HIP library vs CPU oracle)."""
import sys

import numpy as np
import torch

# Tolerance for attention outputs against the oracle: max-abs 2e-2 and
# mean-abs 2e-3 (the bf16-compute contract of the hot path).
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


def assert_close(got, want, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """got: tensor (any float dtype); want: float64 array of the same shape."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - w)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    print(f"[parity] {what}: max_abs={mx:.3e} mean_abs={mean:.3e} n={err.size}", flush=True)
    assert mx <= max_abs, f"{what}: max-abs error {mx:.3e} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean-abs error {mean:.3e} > {mean_abs}"
    return mx, mean
