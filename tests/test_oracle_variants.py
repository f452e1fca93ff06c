"""Pins of the mask and decode variants' oracle against things other than
itself: the base oracle when the window covers everything, torch SDPA with
an explicit banded mask and its autograd, a windowed real prefill behind a
cartridge the window cuts into, finite differences, the closed form of a
one-row window, and a verify step against single decode steps.

Page: "Cartridges: trained KV-prefix corpus compression", sections "gemma4
(measured)" (SWA layers see the cartridge within the window; the window may
cut the prefix) and "Batched self-study (measured)" (multi-token verify
against each stream's own cache).
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import cartattn_oracle as O
from oracle import variants as V
from long_context_kv_amd import workloads as W

TH = W.THETA


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _close(x, ref, tol=1e-12):
    """Normwise error against max(max|ref|, 1): a one-row window makes dQ and
    dK exactly zero in exact arithmetic."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref))) <= tol * max(float(np.max(np.abs(ref))), 1.0)


def _layer(B=2, n=10, p=7, Hq=4, Hkv=2, d=64, seed=3):
    x = W.train_inputs(W.TrainShape("v", B, n, p, Hq, Hkv, d, torch.float32, torch.float32,
                                    seed))
    return [x[k].double().numpy() for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart", "dout")]


def test_visible_window_closed_form():
    vis = V.visible_window(3, 2, 2)
    # query i at position 2 + i sees positions 1 + i and 2 + i
    assert vis.tolist() == [[False, True, True, False, False],
                            [False, False, True, True, False],
                            [False, False, False, True, True]]
    assert V.visible_window(3, 2, 0).sum() == 3 * 2 + 6


@pytest.mark.parametrize("window", [0, 17, 10 ** 6])
def test_wide_window_is_the_base_mask(window):
    q, kt, vt, kc, vc, do = _layer()
    o, l = V.attn_fwd_window(q, kt, vt, kc, vc, window)
    o0, l0 = O.attn_fwd(q, kt, vt, kc, vc)
    assert _rel(o, o0) <= 1e-13 and _rel(l, l0) <= 1e-13
    g = V.attn_bwd_window(q, kt, vt, kc, vc, do, window)
    g0 = O.attn_bwd(q, kt, vt, kc, vc, do)
    for a, b in zip(g, g0):
        assert _rel(a, b) <= 1e-12


@pytest.mark.parametrize("window", [1, 4, 9, 12])
def test_window_matches_sdpa_and_autograd(window):
    q, kt, vt, kc, vc, do = _layer(seed=4)
    B, n, Hq, d = q.shape
    p, Hkv = kc.shape[0], kt.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tkt, tvt = torch.tensor(kt, requires_grad=True), torch.tensor(vt, requires_grad=True)
    tkc, tvc = torch.tensor(kc, requires_grad=True), torch.tensor(vc, requires_grad=True)
    i = torch.arange(n)[:, None] + p
    j = torch.arange(p + n)[None, :]
    mask = (j <= i) & (j > i - window)
    outs = []
    for b in range(B):
        K = torch.cat([tkc, tkt[b]], 0).repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        Vv = torch.cat([tvc, tvt[b]], 0).repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        outs.append(F.scaled_dot_product_attention(tq[b].transpose(0, 1), K, Vv,
                                                   attn_mask=mask).transpose(0, 1))
    o_t = torch.stack(outs)
    (o_t * torch.tensor(do)).sum().backward()
    o, _ = V.attn_fwd_window(q, kt, vt, kc, vc, window)
    assert _rel(o, o_t.detach().numpy()) <= 1e-12
    dq, dkt, dvt, dkc, dvc = V.attn_bwd_window(q, kt, vt, kc, vc, do, window, frozen_rows=0)
    assert _close(dq, tq.grad.numpy())
    assert _close(dkt, tkt.grad.numpy()) and _close(dvt, tvt.grad.numpy())
    assert _close(dkc, tkc.grad.numpy()) and _close(dvc, tvc.grad.numpy())
    # rows the window cuts off for every query get no gradient at all
    first_seen = p - window + 1
    if first_seen > 0:
        assert not np.any(dkc[:first_seen]) and not np.any(dvc[:first_seen])


@pytest.mark.parametrize("window", [3, 8, 20])
def test_window_cutting_the_prefix_equals_windowed_prefill(window):
    """The zero-training gate under a sliding window: the cartridge made of
    the first p rotated rows, behind tokens at p + i, reproduces a windowed
    causal prefill of all p + n rows (rows p..), whether or not the window
    reaches past the cartridge."""
    p, n, Hq, Hkv, d = 8, 12, 4, 2, 64
    q, k, v, _ = [t.double().numpy() for t in W.prefill_raw(p + n, Hq, Hkv, d, 91)]
    pos = O.token_positions(1, p + n, 0)
    qr, kr = O.rope(q, pos, TH), O.rope(k, pos, TH)
    o_full, _ = V.causal_prefill_window(qr, kr, v, window)
    o_c, _ = V.attn_fwd_window(qr[:, p:], kr[:, p:], v[:, p:], kr[0, :p], v[0, :p], window)
    assert _rel(o_c, o_full[:, p:]) <= 1e-12


def test_window_gradients_finite_differences():
    q, kt, vt, kc, vc, do = _layer(B=1, n=5, p=6, seed=5)
    win = 4
    grads = V.attn_bwd_window(q, kt, vt, kc, vc, do, win, frozen_rows=0)
    for which, idx_arr in ((0, q), (3, kc), (4, vc)):
        def f(z):
            args = [q, kt, vt, kc, vc]
            args[which] = z
            return float(np.sum(V.attn_fwd_window(*args, win)[0] * do))
        idx = list(range(0, idx_arr.size, 11))
        fd = O.fd_grad(f, idx_arr, idx)
        got = grads[which].reshape(-1)[idx]
        assert np.max(np.abs(fd - got)) <= 1e-7 * max(1.0, np.max(np.abs(got)))


def test_window_of_one_returns_the_own_value():
    q, kt, vt, kc, vc, _ = _layer(seed=6)
    o, _ = V.attn_fwd_window(q, kt, vt, kc, vc, 1)
    g = q.shape[2] // kt.shape[2]
    assert _rel(o, np.repeat(vt, g, axis=2)) <= 1e-15


def test_verify_equals_sequential_decode_steps():
    g0 = torch.Generator().manual_seed(21)
    S, kq, Hq, Hkv, d = 3, 4, 8, 2, 64
    r = lambda *s: torch.randn(*s, generator=g0, dtype=torch.float32).numpy()
    prefix = [r(5, Hkv, d), r(1, Hkv, d), r(9, Hkv, d)]
    a, b = O.DenseCache(S, Hkv, d), O.DenseCache(S, Hkv, d)
    for s in range(S):
        a.write(s, prefix[s], prefix[s][::-1].copy())
        b.write(s, prefix[s], prefix[s][::-1].copy())
    q, kn, vn = r(S, kq, Hq, d), r(S, kq, Hkv, d), r(S, kq, Hkv, d)
    got = V.verify_step(a, q, kn, vn)
    for t in range(kq):
        ref = O.decode_step(b, q[:, t], kn[:, t], vn[:, t])
        assert _rel(got[:, t], ref) <= 1e-13
    assert [a.seq_len(s) for s in range(S)] == [b.seq_len(s) for s in range(S)]
    c = O.DenseCache(S, Hkv, d)
    for s in range(S):
        c.write(s, prefix[s], prefix[s])
    one = V.verify_step(c, q[:, :1], kn[:, :1], vn[:, :1])
    d2 = O.DenseCache(S, Hkv, d)
    for s in range(S):
        d2.write(s, prefix[s], prefix[s])
    assert _rel(one[:, 0], O.decode_step(d2, q[:, 0], kn[:, 0], vn[:, 0])) <= 1e-15
