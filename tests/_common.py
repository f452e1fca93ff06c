"""Helpers shared by the test modules (no method arithmetic here)."""

import sys

import numpy as np
import torch


def rel(x, ref) -> float:
    """Normwise max error: max|x - ref| / max|ref|."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(x - ref)) / max(den, 1e-300)) if ref.size else 0.0


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (CPU or GPU) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()
