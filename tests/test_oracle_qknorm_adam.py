"""Pins of the oracle for the steps either side of the attention (q/k
RMSNorm + RoPE before it, Adam after it) against things other than itself:
torch's own RMSNorm, RoPE as complex multiplication, torch autograd, finite
differences, torch's Adam, closed forms and invariances.

Page: "Cartridges: trained KV-prefix corpus compression", section
"Semantics (pinned to the reference implementation)" (keys post q/k-norm and
post-RoPE; Adam, no weight decay; frozen row 0) and "Learning rate vs batch
size (measured)".
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import cartattn_oracle as O
from oracle import qknorm_adam as N
from long_context_kv_amd import workloads as W

TH = W.THETA


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _inputs(B=2, S=5, H=3, d=64, seed=7):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, S, H, d, generator=g, dtype=torch.float64) * 3.0
    w = torch.rand(d, generator=g, dtype=torch.float64) + 0.5
    gr = torch.randn(B, S, H, d, generator=g, dtype=torch.float64)
    return x, w, gr


def _torch_norm_rope(x, w, pos, eps):
    """torch's RMSNorm, then RoPE as a complex product: the pair (k, k + d/2)
    is the complex number x_k + i x_{k+d/2}, multiplied by exp(i angle)."""
    d = x.shape[-1]
    y = F.rms_norm(x, (d,), weight=w, eps=eps)
    inv = torch.tensor(TH, dtype=torch.float64) ** (-2.0 * torch.arange(d // 2,
                                                                        dtype=torch.float64) / d)
    ang = torch.as_tensor(pos, dtype=torch.float64)[..., None] * inv        # [B, S, d/2]
    rot = torch.polar(torch.ones_like(ang), ang)[:, :, None, :]            # over heads
    z = torch.complex(y[..., : d // 2], y[..., d // 2:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def test_rms_norm_matches_torch():
    x, w, _ = _inputs()
    for eps in (1e-6, 0.3):
        ref = F.rms_norm(x, (x.shape[-1],), weight=w, eps=eps).numpy()
        assert _rel(N.rms_norm(x.numpy(), w.numpy(), eps), ref) <= 1e-13


def test_rms_norm_closed_form_and_scale_invariance():
    x, _, _ = _inputs()
    xn = x.numpy()
    eps = 0.25
    y = N.rms_norm(xn, np.ones(x.shape[-1]), eps)
    ms = np.mean(xn * xn, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13, atol=0)
    # without eps the output does not depend on the row's scale
    y1 = N.rms_norm(xn, np.ones(x.shape[-1]), 0.0)
    y2 = N.rms_norm(7.5 * xn, np.ones(x.shape[-1]), 0.0)
    assert _rel(y2, y1) <= 1e-14


def test_norm_rope_matches_complex_rotation():
    x, w, _ = _inputs()
    pos = O.token_positions(2, 5, 4096, [0, 300])
    ref = _torch_norm_rope(x, w, pos, 1e-6).numpy()
    assert _rel(N.qk_norm_rope(x.numpy(), w.numpy(), pos, TH, 1e-6), ref) <= 1e-12


def test_norm_rope_bwd_matches_autograd():
    for d in (64, 128):
        x, w, gr = _inputs(d=d, seed=8 + d)
        pos = O.token_positions(2, 5, 17, [3, 0])
        xa = x.clone().requires_grad_(True)
        (_torch_norm_rope(xa, w, pos, 1e-6) * gr).sum().backward()
        got = N.qk_norm_rope_bwd(x.numpy(), w.numpy(), pos, TH, 1e-6, gr.numpy())
        assert _rel(got, xa.grad.numpy()) <= 1e-12


def test_norm_rope_bwd_finite_differences():
    x, w, gr = _inputs(B=1, S=2, H=2, d=64, seed=9)
    xn, wn, gn = x.numpy(), w.numpy(), gr.numpy()
    pos = O.token_positions(1, 2, 40)
    eps = 1e-6
    f = lambda z: float(np.sum(N.qk_norm_rope(z, wn, pos, TH, eps) * gn))
    idx = list(range(0, xn.size, 7))
    fd = O.fd_grad(f, xn, idx)
    got = N.qk_norm_rope_bwd(xn, wn, pos, TH, eps, gn).reshape(-1)[idx]
    assert np.max(np.abs(fd - got)) <= 1e-7 * max(1.0, np.max(np.abs(got)))


def test_norm_rope_bwd_orthogonal_to_input_without_eps():
    """With eps = 0 and w = 1 the output does not change along x (scale
    invariance), so the input gradient of every row is orthogonal to x."""
    x, _, gr = _inputs(seed=10)
    pos = O.token_positions(2, 5, 0)
    dx = N.qk_norm_rope_bwd(x.numpy(), np.ones(64), pos, TH, 0.0, gr.numpy())
    dots = np.sum(dx * x.numpy(), axis=-1)
    assert np.max(np.abs(dots)) <= 1e-12 * np.max(np.abs(dx)) * np.max(np.abs(x.numpy())) * 64


def test_adam_matches_torch_optimizer():
    g0 = torch.Generator().manual_seed(11)
    rows, f = 6, 2
    x = torch.randn(rows, 4, 8, generator=g0, dtype=torch.float64)
    grads = [torch.randn(rows, 4, 8, generator=g0, dtype=torch.float64) for _ in range(3)]
    for lr in (2e-2, 2e-3):
        xn, m, v = x.numpy().copy(), np.zeros_like(x.numpy()), np.zeros_like(x.numpy())
        p = torch.nn.Parameter(x[f:].clone())
        opt = torch.optim.Adam([p], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0)
        for t, g in enumerate(grads, start=1):
            xn, m, v = N.adam_step(xn, g.numpy(), m, v, t, lr, frozen_rows=f)
            p.grad = g[f:].clone()
            opt.step()
            assert _rel(xn[f:], p.detach().numpy()) <= 1e-13
            assert np.array_equal(xn[:f], x.numpy()[:f])          # frozen rows untouched
            st = opt.state[p]
            assert _rel(m[f:], st["exp_avg"].numpy()) <= 1e-13
            assert _rel(v[f:], st["exp_avg_sq"].numpy()) <= 1e-13


def test_adam_first_step_closed_form():
    """At step 1 from zero moments the bias-corrected moments are g and g^2,
    so each parameter moves by -lr g / (|g| + eps)."""
    g0 = torch.Generator().manual_seed(12)
    x = torch.randn(5, 16, generator=g0, dtype=torch.float64).numpy()
    g = torch.randn(5, 16, generator=g0, dtype=torch.float64).numpy()
    z = np.zeros_like(x)
    xn, m, v = N.adam_step(x, g, z, z, 1, 2e-2, frozen_rows=1)
    assert np.allclose(xn[1:] - x[1:], -2e-2 * g[1:] / (np.abs(g[1:]) + 1e-8), rtol=1e-12,
                       atol=1e-17)
    assert np.allclose(m[1:], 0.1 * g[1:], rtol=1e-14) and np.allclose(v[1:], 1e-3 * g[1:] ** 2,
                                                                        rtol=1e-12)
    assert np.array_equal(xn[0], x[0]) and not np.any(m[0]) and not np.any(v[0])
