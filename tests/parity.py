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


def to_gpu(d: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def report(name: str, **errs):
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
