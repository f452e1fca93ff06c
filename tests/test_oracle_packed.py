"""Pins of the packed-segments oracle against things other than itself: one
attention over the whole packed sequence with the block mask (torch SDPA and
autograd), the batched oracle when every segment has the same length,
sequential per-segment training steps accumulating the cartridge gradient,
and RoPE restarting per segment.

Page: "Cartridges: trained KV-prefix corpus compression", sections
"Deliberate divergences from the reference" (packed segments: RoPE restarts
per segment, attention per segment, packed gradients equal sequential ones)
and "Batched self-study (measured)" (one packed forward/backward).
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import cartattn_oracle as O
from oracle import packed as K
from long_context_kv_amd import workloads as W

TH = W.THETA


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _packed(seg_lens, p=6, Hq=4, Hkv=2, d=64, seed=3):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(seg_lens))
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64).numpy()
    return r(T, Hq, d), r(T, Hkv, d), r(T, Hkv, d), r(p, Hkv, d), r(p, Hkv, d), r(T, Hq, d)


def test_offsets_and_positions():
    assert K.seg_offsets([3, 1, 2]).tolist() == [0, 3, 4, 6]
    assert K.packed_positions([3, 1, 2], 10).tolist() == [10, 11, 12, 10, 10, 11]


def test_packed_equals_one_block_masked_attention():
    """The packed forward and its gradients equal a single attention over
    concat(cartridge, all packed tokens) with the block mask (a query sees the
    cartridge and the earlier tokens of its own segment), done by torch."""
    seg = [5, 1, 9, 3]
    q, kt, vt, kc, vc, do = _packed(seg)
    T, Hq, d = q.shape
    p, Hkv = kc.shape[0], kt.shape[1]
    cu = K.seg_offsets(seg)
    segid = np.repeat(np.arange(len(seg)), seg)
    mask = np.zeros((T, p + T), dtype=bool)
    mask[:, :p] = True
    for i in range(T):
        s = segid[i]
        mask[i, p + cu[s]: p + i + 1] = True
    tq, tkt, tvt, tkc, tvc = (torch.tensor(a, requires_grad=True) for a in (q, kt, vt, kc, vc))
    K_ = torch.cat([tkc, tkt], 0).repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
    V_ = torch.cat([tvc, tvt], 0).repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
    o_t = F.scaled_dot_product_attention(tq.transpose(0, 1), K_, V_,
                                         attn_mask=torch.tensor(mask)).transpose(0, 1)
    (o_t * torch.tensor(do)).sum().backward()
    o, _ = K.attn_fwd_packed(q, kt, vt, kc, vc, seg)
    assert _rel(o, o_t.detach().numpy()) <= 1e-12
    dq, dkt, dvt, dkc, dvc = K.attn_bwd_packed(q, kt, vt, kc, vc, do, seg, frozen_rows=0)
    assert _rel(dq, tq.grad.numpy()) <= 1e-12
    assert _rel(dkt, tkt.grad.numpy()) <= 1e-12 and _rel(dvt, tvt.grad.numpy()) <= 1e-12
    assert _rel(dkc, tkc.grad.numpy()) <= 1e-12 and _rel(dvc, tvc.grad.numpy()) <= 1e-12


def test_equal_lengths_equal_the_batched_oracle():
    seg = [7, 7, 7]
    q, kt, vt, kc, vc, do = _packed(seg, seed=4)
    B, n = 3, 7
    rs = lambda a: a.reshape(B, n, *a.shape[1:])
    o, _ = K.attn_fwd_packed(q, kt, vt, kc, vc, seg)
    ob, _ = O.attn_fwd(rs(q), rs(kt), rs(vt), kc, vc)
    assert _rel(o, ob.reshape(o.shape)) <= 1e-13
    g = K.attn_bwd_packed(q, kt, vt, kc, vc, do, seg)
    gb = O.attn_bwd(rs(q), rs(kt), rs(vt), kc, vc, rs(do))
    for a, b in zip(g[:3], gb[:3]):
        assert _rel(a, b.reshape(a.shape)) <= 1e-13
    assert _rel(g[3], gb[3]) <= 1e-13 and _rel(g[4], gb[4]) <= 1e-13


def test_packed_gradient_equals_sequential_accumulation():
    """One packed step == one training step per segment with the cartridge
    gradient accumulated over them (the page's packed-vs-sequential test)."""
    seg = [4, 11, 2]
    q, kt, vt, kc, vc, do = _packed(seg, seed=5)
    g = K.attn_bwd_packed(q, kt, vt, kc, vc, do, seg, frozen_rows=1)
    cu = K.seg_offsets(seg)
    acc_k, acc_v = np.zeros_like(kc), np.zeros_like(vc)
    for s in range(len(seg)):
        r = slice(cu[s], cu[s + 1])
        gs = O.attn_bwd(q[None, r], kt[None, r], vt[None, r], kc, vc, do[None, r], frozen_rows=1)
        assert _rel(g[0][r], gs[0][0]) <= 1e-13
        acc_k += gs[3]
        acc_v += gs[4]
    assert _rel(g[3], acc_k) <= 1e-13 and _rel(g[4], acc_v) <= 1e-13
    assert not np.any(g[3][0]) and not np.any(g[4][0])


def test_rope_restarts_per_segment():
    """Rotating the packed rows at their packed positions equals rotating
    each segment at p + 0, 1, ... on its own."""
    seg = [3, 5]
    g = torch.Generator().manual_seed(6)
    x = torch.randn(8, 2, 64, generator=g, dtype=torch.float64).numpy()
    pos = K.packed_positions(seg, 100)
    rot = O.rope(x[None], pos[None], TH)[0]
    assert _rel(rot[:3], O.rope(x[None, :3], O.token_positions(1, 3, 100), TH)[0]) <= 1e-15
    assert _rel(rot[3:], O.rope(x[None, 3:], O.token_positions(1, 5, 100), TH)[0]) <= 1e-15
