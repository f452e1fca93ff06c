"""Pins of the composition oracle against things other than itself: the
single-cartridge oracle (a one-part composition must equal it bit for bit),
a real causal prefill (two parts split from one capture), torch autograd
through an explicit torch.cat of the parts, and the order invariance of a
fully visible prefix.

Page: "Cartridges: trained KV-prefix corpus compression", section
"Composition" (concatenation; tokens at the composed length; every part
keeps its rotations; gradients reach every part; sinks stay frozen; a single
part equals a single cartridge bitwise; two parts from one capture equal the
real prefill).
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import cartattn_oracle as O
from oracle import composition as P
from long_context_kv_amd import workloads as W

TH = W.THETA


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _parts(rows, Hkv=2, d=64, seed=5):
    g = torch.Generator().manual_seed(seed)
    ks = [torch.randn(r, Hkv, d, generator=g, dtype=torch.float64).numpy() for r in rows]
    vs = [torch.randn(r, Hkv, d, generator=g, dtype=torch.float64).numpy() for r in rows]
    return ks, vs


def _tokens(B=2, n=12, Hq=4, Hkv=2, d=64, seed=6):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64).numpy()
    return r(B, n, Hq, d), r(B, n, Hkv, d), r(B, n, Hkv, d), r(B, n, Hq, d)


def test_composed_p_and_frozen_mask():
    assert P.composed_p([3, 0, 5]) == 8
    m = P.frozen_mask([3, 0, 5], [1, 0, 2])
    assert m.tolist() == [True, False, False, True, True, False, False, False]


def test_single_part_is_the_single_cartridge_bitwise():
    ks, vs = _parts([9])
    q, kt, vt, do = _tokens()
    o1, l1 = P.attn_fwd_composed(q, kt, vt, ks, vs)
    o0, l0 = O.attn_fwd(q, kt, vt, ks[0], vs[0])
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    g1 = P.attn_bwd_composed(q, kt, vt, ks, vs, do, frozen=[1])
    g0 = O.attn_bwd(q, kt, vt, ks[0], vs[0], do, frozen_rows=1)
    for a, b in zip(g1[:3], g0[:3]):
        assert np.array_equal(a, b)
    assert np.array_equal(g1[3][0], g0[3]) and np.array_equal(g1[4][0], g0[4])


def test_two_parts_from_one_capture_equal_the_real_prefill():
    """Rows 0..2p-1 of one capture, rotated at their own positions, split
    into part A (0..p-1) and part B (p..2p-1): behind them the tokens at
    positions 2p + i see exactly what a causal prefill of all rows sees."""
    p, n, Hq, Hkv, d = 6, 10, 4, 2, 64
    q, k, v, dout = [t.double().numpy() for t in W.prefill_raw(2 * p + n, Hq, Hkv, d, 77)]
    T = 2 * p + n
    pos = O.token_positions(1, T, 0)
    qr, kr = O.rope(q, pos, TH), O.rope(k, pos, TH)
    o_full, _ = O.causal_prefill(qr, kr, v)
    parts_k = [kr[0, :p], kr[0, p:2 * p]]
    parts_v = [v[0, :p], v[0, p:2 * p]]
    assert P.composed_p([p, p]) == 2 * p
    tok_pos = O.token_positions(1, n, P.composed_p([p, p]))
    qt, kt = O.rope(q[:, 2 * p:], tok_pos, TH), O.rope(k[:, 2 * p:], tok_pos, TH)
    o_c, _ = P.attn_fwd_composed(qt, kt, v[:, 2 * p:], parts_k, parts_v)
    assert _rel(o_c, o_full[:, 2 * p:]) <= 1e-12
    # gradients: the prefill's with no gradient on the first 2p outputs,
    # except that each part's sink row is frozen
    do = dout.copy()
    do[:, :2 * p] = 0.0
    dq_f, dk_f, dv_f = O.causal_prefill_bwd(qr, kr, v, do)
    dq, dkt, dvt, dkp, dvp = P.attn_bwd_composed(qt, kt, v[:, 2 * p:], parts_k, parts_v,
                                                 dout[:, 2 * p:], frozen=[1, 1])
    assert _rel(dq, dq_f[:, 2 * p:]) <= 1e-12
    assert _rel(dkt, dk_f[:, 2 * p:]) <= 1e-12 and _rel(dvt, dv_f[:, 2 * p:]) <= 1e-12
    for i, (dk, dv) in enumerate(zip(dkp, dvp)):
        rows = slice(i * p, (i + 1) * p)
        assert not np.any(dk[0]) and not np.any(dv[0])             # the part's sink
        assert _rel(dk[1:], dk_f[0, rows][1:]) <= 1e-12
        assert _rel(dv[1:], dv_f[0, rows][1:]) <= 1e-12


def test_gradients_match_autograd_through_an_explicit_cat():
    rows, frozen = [5, 3, 7], [1, 2, 1]
    ks, vs = _parts(rows, seed=8)
    q, kt, vt, do = _tokens(seed=9)
    B, n, Hq, d = q.shape
    Hkv = kt.shape[2]
    tk = [torch.tensor(k, requires_grad=True) for k in ks]
    tv = [torch.tensor(v, requires_grad=True) for v in vs]
    tq = torch.tensor(q, requires_grad=True)
    tkt = torch.tensor(kt, requires_grad=True)
    tvt = torch.tensor(vt, requires_grad=True)
    Pn = sum(rows)
    out = []
    for b in range(B):
        K = torch.cat(tk + [tkt[b]], 0).repeat_interleave(Hq // Hkv, dim=1)   # [L, Hq, d]
        V = torch.cat(tv + [tvt[b]], 0).repeat_interleave(Hq // Hkv, dim=1)
        mask = torch.arange(Pn + n)[None, :] <= (torch.arange(n)[:, None] + Pn)
        o = F.scaled_dot_product_attention(tq[b].transpose(0, 1), K.transpose(0, 1),
                                           V.transpose(0, 1), attn_mask=mask)
        out.append(o.transpose(0, 1))
    (torch.stack(out) * torch.tensor(do)).sum().backward()
    dq, dkt, dvt, dkp, dvp = P.attn_bwd_composed(q, kt, vt, ks, vs, do, frozen)
    assert _rel(dq, tq.grad.numpy()) <= 1e-12
    assert _rel(dkt, tkt.grad.numpy()) <= 1e-12 and _rel(dvt, tvt.grad.numpy()) <= 1e-12
    for i, f in enumerate(frozen):
        gk, gv = tk[i].grad.numpy(), tv[i].grad.numpy()
        assert np.any(gk[:f]) and not np.any(dkp[i][:f]) and not np.any(dvp[i][:f])
        assert _rel(dkp[i][f:], gk[f:]) <= 1e-12 and _rel(dvp[i][f:], gv[f:]) <= 1e-12
        assert np.any(dkp[i][f:]) and np.any(dvp[i][f:])          # every part learns


def test_part_order_does_not_change_the_output():
    """Every prefix row is visible to every query, so the composed prefix
    acts as a set: swapping the parts leaves O unchanged and swaps the parts'
    gradients."""
    ks, vs = _parts([4, 6], seed=10)
    q, kt, vt, do = _tokens(seed=11)
    o_ab, _ = P.attn_fwd_composed(q, kt, vt, ks, vs)
    o_ba, _ = P.attn_fwd_composed(q, kt, vt, ks[::-1], vs[::-1])
    assert _rel(o_ba, o_ab) <= 1e-12
    g_ab = P.attn_bwd_composed(q, kt, vt, ks, vs, do, [1, 1])
    g_ba = P.attn_bwd_composed(q, kt, vt, ks[::-1], vs[::-1], do, [1, 1])
    assert _rel(g_ba[3][1], g_ab[3][0]) <= 1e-12 and _rel(g_ba[4][0], g_ab[4][1]) <= 1e-12
