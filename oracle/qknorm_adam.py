"""Plain CPU float64 oracle for the steps either side of the attention:
the q/k RMS normalization + RoPE before it and Adam on the cartridge rows
after it.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module. It shares no code with the GPU path.

Sources (titles of the pages the method is described on):

* "Cartridges: trained KV-prefix corpus compression" (Fucina guide), section
  "Semantics (pinned to the reference implementation)": cartridge keys are
  KV-cache rows taken after the q/k normalization and after RoPE, so real
  tokens' queries and keys enter the attention normalized and then rotated
  at positions p, p+1, ...; the rows below frozen_prefix are constants and
  the rest are optimized by Adam with no weight decay and no schedule
  (lr 2e-2). Section "Learning rate vs batch size (measured)": lr 2e-3 at
  small batches.

Readings where the pages are silent:

* the normalization is the Qwen3 q/k RMSNorm over one head row with a
  learned weight: y = x * w / sqrt(mean(x^2) + eps) (eps 1e-6 for Qwen3);
  the weights are frozen, so only the input gradient is formed;
* Adam is the bias-corrected Adam of Kingma and Ba with the betas and eps
  of the common defaults (0.9, 0.999, 1e-8), eps added after the square root
  of the bias-corrected second moment; frozen rows keep their value and
  their moments.
"""

from __future__ import annotations

import numpy as np

from oracle.cartattn_oracle import rope

__all__ = ["rms_norm", "qk_norm_rope", "qk_norm_rope_bwd", "adam_step"]


def rms_norm(x, w, eps: float):
    """y = x * w / sqrt(mean(x^2) + eps) over the last axis (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * w / np.sqrt(ms + eps)


def qk_norm_rope(x, w, positions, theta: float, eps: float):
    """Normalize each head row of x [..., S, H, d], then rotate it at
    positions[..., S] (the rotation of ``rope``)."""
    return rope(rms_norm(x, w, eps), positions, theta)


def qk_norm_rope_bwd(x, w, positions, theta: float, eps: float, g):
    """Gradient with respect to x of sum(qk_norm_rope(x) * g).

    The rotation is orthogonal, so its adjoint is the rotation by -angle:
    dy = rope(g, inverse=True). For y = x w r with r = (mean(x^2) + eps)^(-1/2),
    dr/dx_k = -r^3 x_k / d, hence
    dx_k = r w_k dy_k - (r^3 / d) x_k sum_j w_j dy_j x_j.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    d = x.shape[-1]
    dy = rope(g, positions, theta, inverse=True)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    t = np.sum(w * dy * x, axis=-1, keepdims=True)
    return r * w * dy - (r ** 3 / d) * x * t


def adam_step(x, g, m, v, step: int, lr: float, beta1: float = 0.9,
              beta2: float = 0.999, eps: float = 1e-8, frozen_rows: int = 0):
    """One bias-corrected Adam step on rows >= frozen_rows of x [rows, ...].

    Returns new (x, m, v) as float64 arrays; rows below frozen_rows are
    returned unchanged.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    g = np.asarray(g, np.float64)
    m = np.array(m, dtype=np.float64, copy=True)
    v = np.array(v, dtype=np.float64, copy=True)
    f = int(frozen_rows)
    m_new = beta1 * m[f:] + (1.0 - beta1) * g[f:]
    v_new = beta2 * v[f:] + (1.0 - beta2) * g[f:] * g[f:]
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    x[f:] = x[f:] - lr * m_hat / (np.sqrt(v_hat) + eps)
    m[f:] = m_new
    v[f:] = v_new
    return x, m, v
