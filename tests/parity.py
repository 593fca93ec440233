"""Helpers for GPU-vs-oracle parity checks.

Acceptance bound: max|x - x_ref| / RMS(x_ref) over a whole tensor, with
RMS(x) = sqrt(mean(x^2)).  1e-4 for fp32 inputs, 2e-2 for bf16 inputs with
fp32 accumulation; the same bounds apply to the final states.
"""

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, ref) -> float:
    x = x.detach().cpu().double().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref))) / rms if x.size else 0.0


def rel_err_rounded(x, ref, ulp_rel: float) -> float:
    """rel_err for an output stored in a narrower format: each element may
    also carry that format's own rounding, up to ulp_rel |ref| (half an ulp of
    bf16 is 2^-9 of the value; 2^-8 covers the kernel's own error moving an
    element across a rounding boundary)."""
    x = x.detach().cpu().double().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    rms = float(np.sqrt(np.mean(ref * ref)))
    if not x.size:
        return 0.0
    excess = np.maximum(np.abs(x - ref) - ulp_rel * np.abs(ref), 0.0)
    return float(np.max(excess)) / (rms if rms > 0.0 else 1.0)


def to_gpu(d: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def report(name: str, **errs):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


class StreamErr:
    """max|x - x_ref| / RMS(x_ref) over a tensor compared piece by piece: the
    maximum and the sum of squares are accumulated over the pieces, so the
    ratio is the one over the whole tensor."""

    def __init__(self):
        self.max_abs = 0.0
        self.sumsq = 0.0
        self.count = 0

    def update(self, x, ref):
        x = x.detach().cpu().double().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
        ref = np.asarray(ref, np.float64)
        assert x.shape == ref.shape, (x.shape, ref.shape)
        assert np.all(np.isfinite(x)), "non-finite values in GPU output"
        if x.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(x - ref))))
            self.sumsq += float(np.sum(ref * ref))
            self.count += ref.size

    def value(self) -> float:
        rms = float(np.sqrt(self.sumsq / self.count)) if self.count else 0.0
        return self.max_abs / rms if rms > 0.0 else self.max_abs
