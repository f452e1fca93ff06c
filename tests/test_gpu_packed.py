"""GPU parity of packed segments behind one cartridge (varlen tokens: each
segment attends causally over itself behind the shared prefix, RoPE
restarting per segment, one summed cartridge gradient) through the C ABI,
against the packed oracle.

Page: "Cartridges: trained KV-prefix corpus compression", section
"Deliberate divergences from the reference" (packed segments; packed vs
sequential gradient equality) and "Batched self-study (measured)".
"""

import numpy as np
import pytest
import torch

from oracle import cartattn_oracle as O
from oracle import packed as K
from oracle import variants as V
from long_context_kv_amd import workloads as W
from tests._common import f64, rel, say

pytestmark = pytest.mark.gpu

TH = W.THETA


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_kv_amd import cartattn
    return cartattn


def _packed_inputs(seg, p, Hq, Hkv, d, tok, row, seed):
    T = int(sum(seg))
    x = W.train_inputs(W.TrainShape("pk", 1, T, p, Hq, Hkv, d, tok, row, seed))
    return {k: (v[0] if k in ("q", "k_tok", "v_tok", "dout") else v) for k, v in x.items()}


def _gpu(C, x, seg, p, f, window=0):
    g = {k: v.cuda().contiguous() for k, v in x.items()}
    kc = g["k_cart"] if p else None
    vc = g["v_cart"] if p else None
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], kc, vc, frozen_rows=f, seg_lens=seg,
                        window=window)
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], kc, vc, o, lse, g["dout"], frozen_rows=f,
                       seg_lens=seg, window=window)
    torch.cuda.synchronize()
    return o, lse, grads


def _compare(o, grads, x, seg, p, f, tol, window=0):
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    if window == 0:
        o_ref, _ = K.attn_fwd_packed(*args, seg)
        ref = K.attn_bwd_packed(*args, f64(x["dout"]), seg, frozen_rows=f)
    else:
        # the window oracle per segment (each segment is one sequence)
        cu = K.seg_offsets(seg)
        o_ref = np.zeros(args[0].shape)
        ref = [np.zeros(args[0].shape), np.zeros(args[1].shape), np.zeros(args[2].shape),
               np.zeros(args[3].shape), np.zeros(args[4].shape)]
        for s in range(len(seg)):
            r = slice(cu[s], cu[s + 1])
            a_s = [args[0][None, r], args[1][None, r], args[2][None, r], args[3], args[4]]
            o_ref[r] = V.attn_fwd_window(*a_s, window)[0][0]
            g_s = V.attn_bwd_window(*a_s, f64(x["dout"])[None, r], window, frozen_rows=0)
            for t in range(3):
                ref[t][r] = g_s[t][0]
            ref[3] += g_s[3]
            ref[4] += g_s[4]
        ref[3][:f] = 0
        ref[4][:f] = 0
    errs = {"o": rel(f64(o), o_ref)}
    for name, gpu, r in zip(("dq", "dk_tok", "dv_tok"), grads[:3], ref[:3]):
        errs[name] = rel(f64(gpu), r)
    if p:
        for name, gpu, r in zip(("dk_cart", "dv_cart"), grads[3:], ref[3:]):
            gg = f64(gpu)
            assert np.all(gg[:f] == 0), name
            errs[name] = rel(gg[f:], r[f:])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, errs
    return errs


CASES = [
    # name, seg lens, p, Hq, Hkv, d
    ("ragged-g4", [77, 1, 200, 33, 128], 300, 8, 2, 128),
    ("ragged-d64", [64, 150, 9], 130, 6, 3, 64),
    ("many-short", [5, 17, 3, 31, 32, 33, 1, 64, 2, 40], 64, 4, 2, 128),
    ("no-cart", [50, 100], 0, 4, 4, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_bf16(C, case):
    name, seg, p, Hq, Hkv, d = case
    f = min(1, p)
    x = _packed_inputs(seg, p, Hq, Hkv, d, torch.bfloat16, torch.float32, 81)
    say("packed bf16", name)
    o, _, grads = _gpu(C, x, seg, p, f)
    say("errors", _compare(o, grads, x, seg, p, f, 2e-2))


def test_packed_f32(C):
    seg = [9, 1, 14]
    x = _packed_inputs(seg, 12, 4, 2, 64, torch.float32, torch.float32, 82)
    say("packed f32")
    o, _, grads = _gpu(C, x, seg, 12, 1)
    _compare(o, grads, x, seg, 12, 1, 1e-5)


def test_packed_with_window(C):
    seg = [120, 7, 260]
    x = _packed_inputs(seg, 200, 8, 2, 128, torch.bfloat16, torch.float32, 83)
    say("packed + window")
    o, _, grads = _gpu(C, x, seg, 200, 1, window=90)
    _compare(o, grads, x, seg, 200, 1, 2e-2, window=90)


def test_equal_lengths_equal_the_batch_bitwise(C):
    """Packed segments of one length run the same work as the batch."""
    B, n, p = 3, 96, 200
    sh = W.TrainShape("eq", B, n, p, 8, 2, 128, torch.bfloat16, torch.float32, 84)
    x = W.train_inputs(sh)
    g = {k: v.cuda() for k, v in x.items()}
    say("packed == batch")
    ob, lb = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"])
    gb = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], ob, lb, g["dout"])
    flat = lambda t: t.reshape(B * n, *t.shape[2:]).contiguous()
    op, lp = C.attn_fwd(flat(g["q"]), flat(g["k_tok"]), flat(g["v_tok"]), g["k_cart"],
                        g["v_cart"], seg_lens=[n] * B)
    gp = C.attn_bwd(flat(g["q"]), flat(g["k_tok"]), flat(g["v_tok"]), g["k_cart"], g["v_cart"],
                    op, lp, flat(g["dout"]), seg_lens=[n] * B)
    torch.cuda.synchronize()
    assert torch.equal(op, flat(ob)) and torch.equal(lp, lb)
    for a, b in zip(gp[:3], gb[:3]):
        assert torch.equal(a, flat(b))
    assert torch.equal(gp[3], gb[3]) and torch.equal(gp[4], gb[4])


def test_packed_equals_sequential_steps(C):
    """One packed step == one step per segment with the cartridge gradient
    accumulated (accumulate_cart) over them."""
    seg = [40, 130, 65]
    x = _packed_inputs(seg, 150, 8, 2, 128, torch.bfloat16, torch.float32, 85)
    g = {k: v.cuda().contiguous() for k, v in x.items()}
    say("packed vs sequential")
    o, _, gp = _gpu(C, x, seg, 150, 1)
    cu = K.seg_offsets(seg)
    dkc = torch.zeros_like(gp[3])
    dvc = torch.zeros_like(gp[4])
    for s in range(len(seg)):
        r = slice(int(cu[s]), int(cu[s + 1]))
        one = lambda t: t[r][None].contiguous()
        os_, ls_ = C.attn_fwd(one(g["q"]), one(g["k_tok"]), one(g["v_tok"]), g["k_cart"],
                              g["v_cart"])
        gs = C.attn_bwd(one(g["q"]), one(g["k_tok"]), one(g["v_tok"]), g["k_cart"], g["v_cart"],
                        os_, ls_, one(g["dout"]), dk_cart=dkc, dv_cart=dvc,
                        accumulate_cart=s > 0)
        torch.cuda.synchronize()
        # the same rows and products; only the key-split of the forward (and
        # so the rounding order) may differ between the two launches
        assert rel(f64(os_[0]), f64(o[r])) <= 1e-2
        assert rel(f64(gs[0][0]), f64(gp[0][r])) <= 1e-2
    assert rel(f64(dkc)[1:], f64(gp[3])[1:]) <= 1e-4 and rel(f64(dvc)[1:], f64(gp[4])[1:]) <= 1e-4


def test_rope_packed(C):
    seg = [5, 40, 1, 19]
    T = sum(seg)
    g0 = torch.Generator().manual_seed(86)
    q = torch.randn(T, 6, 128, generator=g0).to(torch.bfloat16)
    k = torch.randn(T, 2, 128, generator=g0).to(torch.bfloat16)
    qd, kd = q.cuda(), k.cuda()
    say("rope packed")
    C.cart_rope_tokens_packed(qd, kd, seg, pos_base=300, theta=TH)
    torch.cuda.synchronize()
    pos = K.packed_positions(seg, 300)
    assert rel(f64(qd), O.rope(f64(q)[None], pos[None], TH)[0]) <= 2e-2
    # each segment as its own sequence: the same bits
    cu = K.seg_offsets(seg)
    for s in range(len(seg)):
        qs = q[cu[s]:cu[s + 1]][None].cuda().contiguous()
        ks = k[cu[s]:cu[s + 1]][None].cuda().contiguous()
        C.cart_rope_tokens(qs, ks, pos_base=300, theta=TH)
        torch.cuda.synchronize()
        assert torch.equal(qs[0], qd[cu[s]:cu[s + 1]]) and torch.equal(ks[0], kd[cu[s]:cu[s + 1]])


def test_packed_long_cartridge_layer(C):
    """The long-cartridge layer's 4096 tokens as four packed segments behind
    p = 16384: two kv heads compared with the oracle."""
    sh = W.LONG
    seg = [1024, 512, 2048, 512]
    x = W.train_inputs(sh, seed=sh.seed)
    x = {k: (v[0] if k in ("q", "k_tok", "v_tok", "dout") else v) for k, v in x.items()}
    say("packed long-cartridge layer")
    o, _, grads = _gpu(C, x, seg, sh.p, 1)
    o, grads = o.cpu(), [t.cpu() for t in grads]
    kvh = [0, 7]
    qh = [kv * 2 + j for kv in kvh for j in range(2)]
    xs = dict(q=x["q"][:, qh], k_tok=x["k_tok"][:, kvh], v_tok=x["v_tok"][:, kvh],
              k_cart=x["k_cart"][:, kvh], v_cart=x["v_cart"][:, kvh], dout=x["dout"][:, qh])
    gs = (grads[0][:, qh], grads[1][:, kvh], grads[2][:, kvh], grads[3][:, kvh], grads[4][:, kvh])
    say("oracle on kv heads", kvh)
    say("errors", _compare(o[:, qh], gs, xs, seg, sh.p, 1, 2e-2))
