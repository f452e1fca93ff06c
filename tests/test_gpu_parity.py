"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle.

Tolerances: max normwise relative error 1e-5 in the float32 reference mode,
2e-2 for bf16 inputs; frozen cartridge rows must be exactly zero. Every
input comes from the seeded generators; every expected value comes from the
oracle on the same inputs.
"""

import numpy as np
import pytest
import torch

from oracle import cartattn_oracle as O
from long_context_kv_amd import workloads as W
from tests._common import f64, rel, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TH = W.THETA


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_kv_amd import cartattn
    return cartattn


def _dev(x):
    return {k: v.cuda().contiguous() for k, v in x.items()}


def _shape(name, B, n, p, Hq, Hkv, d, tok, row, seed):
    return W.TrainShape(name, B, n, p, Hq, Hkv, d, tok, row, seed)


def _oracle_step(x, p, f, tok_rotated=None):
    """Oracle over raw inputs: RoPE at p + i, forward, backward, RoPE adjoint."""
    q, kt = f64(x["q"]), f64(x["k_tok"])
    B, n = q.shape[:2]
    pos = O.token_positions(B, n, p)
    qr = O.rope(q, pos, TH)
    kr = O.rope(kt, pos, TH)
    vt, kc, vc, do = f64(x["v_tok"]), f64(x["k_cart"]), f64(x["v_cart"]), f64(x["dout"])
    o, lse = O.attn_fwd(qr, kr, vt, kc, vc)
    dq, dkt, dvt, dkc, dvc = O.attn_bwd(qr, kr, vt, kc, vc, do, frozen_rows=f)
    dq = O.rope(dq, pos, TH, inverse=True)
    dkt = O.rope(dkt, pos, TH, inverse=True)
    return dict(o=o, lse=lse, dq=dq, dk_tok=dkt, dv_tok=dvt, dk_cart=dkc, dv_cart=dvc)


def _gpu_step(C, x, p, f):
    """The hot path on the GPU: RoPE, forward, backward, RoPE adjoint."""
    g = _dev(x)
    q, kt = g["q"].clone(), g["k_tok"].clone()
    C.cart_rope_tokens(q, kt, pos_base=p, theta=TH)
    o, lse = C.attn_fwd(q, kt, g["v_tok"], g["k_cart"], g["v_cart"], frozen_rows=f)
    dq, dkt, dvt, dkc, dvc = C.attn_bwd(q, kt, g["v_tok"], g["k_cart"], g["v_cart"], o, lse,
                                        g["dout"], frozen_rows=f)
    C.cart_rope_tokens(dq, dkt, pos_base=p, theta=TH, inverse=True)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, dq=dq, dk_tok=dkt, dv_tok=dvt, dk_cart=dkc, dv_cart=dvc)


def _compare(got, ref, tol, f, names=("o", "dq", "dk_tok", "dv_tok", "dk_cart", "dv_cart")):
    errs = {}
    for k in names:
        if ref[k] is None or ref[k].size == 0:
            continue
        g = f64(got[k])
        if k in ("dk_cart", "dv_cart") and f > 0:
            assert np.all(g[:f] == 0.0), f"{k}: frozen rows not exactly zero"
            errs[k] = rel(g[f:], ref[k][f:])
        else:
            errs[k] = rel(g, ref[k])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {errs}"
    return errs


# ------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_rope_parity(C, dtype, d):
    say("rope", dtype, d)
    sh = _shape("r", 3, 37, 0, 6, 2, d, dtype, dtype, 41)
    x = W.train_inputs(sh)
    offs = torch.tensor([0, 5, 4096], dtype=torch.int32)
    q, k = x["q"].cuda(), x["k_tok"].cuda()
    C.cart_rope_tokens(q, k, pos_base=2048, pos_offsets=offs.cuda(), theta=TH)
    torch.cuda.synchronize()
    pos = O.token_positions(3, 37, 2048, offs.numpy())
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    assert rel(f64(q), O.rope(f64(x["q"]), pos, TH)) <= tol
    assert rel(f64(k), O.rope(f64(x["k_tok"]), pos, TH)) <= tol
    C.cart_rope_tokens(q, k, pos_base=2048, pos_offsets=offs.cuda(), theta=TH, inverse=True)
    torch.cuda.synchronize()
    back_tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert rel(f64(q), f64(x["q"])) <= back_tol
    # position 0 is the identity, bit for bit
    q0 = x["q"][:, :1].contiguous().cuda()
    C.cart_rope_tokens(q0, None, pos_base=0, theta=TH)
    torch.cuda.synchronize()
    assert torch.equal(q0.cpu(), x["q"][:, :1])


# ----------------------------------------------- float32 reference mode (tiny)

def test_tiny_f32_full_step(C):
    say("tiny f32 full step")
    sh = W.TINY
    x = W.train_inputs(sh)
    ref = _oracle_step(x, sh.p, sh.frozen_rows)
    got = _gpu_step(C, x, sh.p, sh.frozen_rows)
    _compare(got, ref, TOL_F32, sh.frozen_rows)
    assert rel(f64(got["lse"]), ref["lse"]) <= TOL_F32


def test_tiny_f32_prefill_equivalence(C):
    """Zero-training gate on the GPU: a cartridge built from the first p rotated
    rows reproduces a p = 0 causal prefill of all p + n rows (rows p..)."""
    say("tiny f32 prefill equivalence")
    p, n, Hq, Hkv, d = 8, 16, 4, 2, 64
    q, k, v, _ = W.prefill_raw(p + n, Hq, Hkv, d, 101)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    C.cart_rope_tokens(qg, kg, pos_base=0, theta=TH)          # all T rows at 0..T-1
    o_full, _ = C.attn_fwd(qg, kg, vg, None, None, frozen_rows=0)
    k_cart = kg[0, :p].contiguous()
    v_cart = vg[0, :p].contiguous()
    qt, kt = q[:, p:].cuda().contiguous(), k[:, p:].cuda().contiguous()
    C.cart_rope_tokens(qt, kt, pos_base=p, theta=TH)
    o_c, _ = C.attn_fwd(qt, kt, vg[:, p:].contiguous(), k_cart, v_cart, frozen_rows=1)
    torch.cuda.synchronize()
    assert rel(f64(o_c), f64(o_full[:, p:])) <= TOL_F32
    ref, _ = O.causal_prefill(O.rope(f64(q), O.token_positions(1, p + n, 0), TH),
                              O.rope(f64(k), O.token_positions(1, p + n, 0), TH), f64(v))
    assert rel(f64(o_c), ref[:, p:]) <= TOL_F32


# ------------------------------------- kernel parity on identical inputs

SMALL = [
    # name, B, n, p, Hq, Hkv, d
    ("ragged-g4", 2, 77, 200, 8, 2, 128),
    ("g2-d64", 3, 33, 65, 6, 3, 64),
    ("mha-no-cart", 1, 100, 0, 4, 4, 64),
    ("g8", 1, 70, 130, 16, 2, 128),
    ("g1-long-p", 1, 40, 700, 2, 2, 128),
    ("one-token", 2, 1, 9, 4, 2, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("mode", ["f32", "bf16-f32rows", "bf16-bf16rows"])
def test_attention_parity_small(C, case, mode):
    name, B, n, p, Hq, Hkv, d = case
    tok = torch.float32 if mode == "f32" else torch.bfloat16
    row = torch.bfloat16 if mode == "bf16-bf16rows" else torch.float32
    say("attention", name, mode)
    f = min(1, p)
    x = W.train_inputs(_shape(name, B, n, p, Hq, Hkv, d, tok, row, 77))
    g = _dev(x)
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"] if p else None,
                        g["v_cart"] if p else None, frozen_rows=f)
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"] if p else None,
                       g["v_cart"] if p else None, o, lse, g["dout"], frozen_rows=f)
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, lse_ref = O.attn_fwd(*args)
    gr = O.attn_bwd(*args, f64(x["dout"]), frozen_rows=f)
    got = dict(o=o, dq=grads[0], dk_tok=grads[1], dv_tok=grads[2], dk_cart=grads[3],
               dv_cart=grads[4])
    ref = dict(o=o_ref, dq=gr[0], dk_tok=gr[1], dv_tok=gr[2], dk_cart=gr[3] if p else None,
               dv_cart=gr[4] if p else None)
    tol = TOL_F32 if mode == "f32" else TOL_BF16
    _compare(got, ref, tol, f, names=[k for k in ref if ref[k] is not None])
    assert np.max(np.abs(f64(lse) - lse_ref)) <= (1e-5 if mode == "f32" else 2e-2)


# Shapes that give the dK/dV kernel's software pipeline pieces of 1, 2, 3 and
# many units, ragged query tiles, GQA groups of 1 to 4, key tiles cut into
# pieces (reduced in the kernel) and token-heavy grids.
PIPELINE = [
    # name, B, n, p, Hq, Hkv, d
    ("units-1", 1, 20, 100, 1, 1, 128),
    ("units-2", 1, 40, 130, 2, 1, 128),
    ("units-3-ragged", 1, 70, 260, 3, 1, 128),
    ("pieces-g4", 2, 200, 600, 8, 2, 128),
    ("pieces-d64", 2, 150, 500, 8, 2, 64),
    ("token-heavy", 1, 500, 16, 4, 2, 128),
]


@pytest.mark.parametrize("case", PIPELINE, ids=[c[0] for c in PIPELINE])
def test_attention_parity_pipeline_edges(C, case):
    name, B, n, p, Hq, Hkv, d = case
    say("pipeline", name)
    x = W.train_inputs(_shape(name, B, n, p, Hq, Hkv, d, torch.bfloat16, torch.float32, 91))
    g = _dev(x)
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], frozen_rows=1)
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], o, lse, g["dout"],
                       frozen_rows=1)
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, _ = O.attn_fwd(*args)
    gr = O.attn_bwd(*args, f64(x["dout"]), frozen_rows=1)
    got = dict(o=o, dq=grads[0], dk_tok=grads[1], dv_tok=grads[2], dk_cart=grads[3],
               dv_cart=grads[4])
    ref = dict(o=o_ref, dq=gr[0], dk_tok=gr[1], dv_tok=gr[2], dk_cart=gr[3], dv_cart=gr[4])
    _compare(got, ref, TOL_BF16, 1)


def test_peaked_softmax_and_accumulate(C):
    """Sharper scores (q x 4) stress the online-softmax rescaling; a second
    backward with accumulate_cart adds into the cartridge gradients."""
    say("peaked + accumulate")
    sh = _shape("peak", 2, 96, 160, 8, 2, 128, torch.bfloat16, torch.float32, 5)
    x = W.train_inputs(sh, q_scale=4.0)
    g = _dev(x)
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"])
    gr1 = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], o, lse, g["dout"])
    dkc = gr1[3].clone()
    dvc = gr1[4].clone()
    C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], o, lse, g["dout"],
               dk_cart=dkc, dv_cart=dvc, accumulate_cart=True)
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, _ = O.attn_fwd(*args)
    ref = O.attn_bwd(*args, f64(x["dout"]), frozen_rows=1)
    assert rel(f64(o), o_ref) <= TOL_BF16
    for t in range(5):
        assert rel(f64(gr1[t]), ref[t]) <= TOL_BF16, t
    assert np.all(f64(dkc)[0] == 0) and np.all(f64(dvc)[0] == 0)
    assert rel(f64(dkc)[1:], 2 * ref[3][1:]) <= TOL_BF16
    assert rel(f64(dvc)[1:], 2 * ref[4][1:]) <= TOL_BF16


def test_invariants_on_gpu(C):
    """Sum of dV over all rows = sum of dO over the group; sum of dK = 0."""
    say("invariants")
    sh = _shape("inv", 2, 64, 96, 8, 2, 128, torch.bfloat16, torch.float32, 8)
    x = W.train_inputs(sh)
    g = _dev(x)
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], frozen_rows=0)
    dq, dkt, dvt, dkc, dvc = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"],
                                        g["v_cart"], o, lse, g["dout"], frozen_rows=0)
    torch.cuda.synchronize()
    do = f64(x["dout"])
    for kv in range(2):
        sdv = f64(dvc)[:, kv].sum(0) + f64(dvt)[:, :, kv].sum((0, 1))
        sdo = do[:, :, 4 * kv:4 * kv + 4].sum((0, 1, 2))
        assert rel(sdv, sdo) <= TOL_BF16
        sdk = f64(dkc)[:, kv].sum(0) + f64(dkt)[:, :, kv].sum((0, 1))
        scale = np.abs(f64(dkc)[:, kv]).sum(0).max()
        assert np.max(np.abs(sdk)) <= 2e-2 * scale


# ------------------------------------------------------- full-size configs

def _heads_subset(x, kv_heads, g):
    """Restrict a layer's inputs to some kv heads (heads are independent)."""
    qh = [kv * g + j for kv in kv_heads for j in range(g)]
    out = dict(x)
    out["q"] = x["q"][:, :, qh]
    out["dout"] = x["dout"][:, :, qh]
    for k in ("k_tok", "v_tok"):
        out[k] = x[k][:, :, kv_heads]
    for k in ("k_cart", "v_cart"):
        out[k] = x[k][:, kv_heads]
    return out, qh


_FULL = {}


def _full_gpu(C, sh, seed):
    """GPU outputs of one full-size layer, computed once per (shape, seed)."""
    key = (sh.name, seed)
    if key not in _FULL:
        _FULL.clear()                       # keep one layer's outputs at a time
        x = W.train_inputs(sh, seed=seed)
        say(sh.name, "seed", seed, "GPU step")
        got = _gpu_step(C, x, sh.p, sh.frozen_rows)
        _FULL[key] = (x, {k: v.cpu() for k, v in got.items()})
    return _FULL[key]


def _full_config(C, sh, seed, kv_heads):
    x, got = _full_gpu(C, sh, seed)
    g = sh.n_q_heads // sh.n_kv_heads
    xs, qh = _heads_subset(x, kv_heads, g)
    say(sh.name, "seed", seed, "oracle on kv heads", kv_heads)
    ref = _oracle_step(xs, sh.p, sh.frozen_rows)
    sub = dict(o=got["o"][:, :, qh], dq=got["dq"][:, :, qh], dk_tok=got["dk_tok"][:, :, kv_heads],
               dv_tok=got["dv_tok"][:, :, kv_heads], dk_cart=got["dk_cart"][:, kv_heads],
               dv_cart=got["dv_cart"][:, kv_heads])
    return _compare(sub, ref, TOL_BF16, sh.frozen_rows)


# Every kv head of every full-size layer meets the oracle; the heads are
# compared in two halves so that each test stays well under a minute of
# oracle time on the host.
HALVES = [list(range(0, 4)), list(range(4, 8))]


def test_config_qwen3_0_6b_layer(C):
    errs = _full_config(C, W.QWEN3_0_6B, W.QWEN3_0_6B.seed, list(range(8)))
    say("errors", errs)


@pytest.mark.parametrize("half", [0, 1])
def test_config_qwen3_8b_layer(C, half):
    errs = _full_config(C, W.QWEN3_8B, W.QWEN3_8B.seed, HALVES[half])
    say("errors", errs)


@pytest.mark.parametrize("half", [0, 1])
@pytest.mark.parametrize("layer", [0, 27])
def test_config_long_cartridge_layer(C, layer, half):
    errs = _full_config(C, W.LONG, W.LONG.seed + layer, HALVES[half])
    say("errors", errs)


# ------------------------------------------------------ invariants / edges

def test_frozen_rows_three(C):
    """frozen_rows = 3: rows 0..2 of both cartridge gradients are exactly zero
    (the unfrozen gradient there is not), the rest match the oracle."""
    sh = W.TrainShape("frozen3", 2, 90, 150, 8, 2, 128, torch.bfloat16, torch.float32, 13,
                      frozen_rows=3)
    x = W.train_inputs(sh)
    say("frozen rows 3")
    got = _gpu_step(C, x, sh.p, 3)
    ref = _oracle_step(x, sh.p, 3)
    _compare(got, ref, TOL_BF16, 3)
    free = _oracle_step(x, sh.p, 0)
    assert np.max(np.abs(free["dk_cart"][:3])) > 0 and np.max(np.abs(free["dv_cart"][:3])) > 0


@pytest.mark.parametrize("case", [("pieces-g4", 2, 200, 600, 8, 2, 128),
                                  ("qwen3-0.6b-layer", 1, 1024, 2048, 16, 8, 128)],
                         ids=["pieces-g4", "qwen3-0.6b-layer"])
def test_bf16_repeat_run_is_bitwise(C, case):
    """The bf16 path takes no float atomics (cut tiles and key splits are
    summed in a fixed order), so two runs on the same inputs agree bit for bit."""
    name, B, n, p, Hq, Hkv, d = case
    sh = _shape(name, B, n, p, Hq, Hkv, d, torch.bfloat16, torch.float32, 17)
    x = W.train_inputs(sh)
    say("repeat run", name)
    a = _gpu_step(C, x, p, 1)
    b = _gpu_step(C, x, p, 1)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_key_shift_invariance(C):
    """Adding one vector c to every key row (cartridge and token) shifts each
    query's scores by q.c, which the softmax removes: O and every gradient are
    unchanged. The GPU run on shifted keys matches the oracle on the
    unshifted ones."""
    sh = _shape("shift", 2, 80, 140, 8, 2, 128, torch.bfloat16, torch.float32, 23)
    x = W.train_inputs(sh)
    c = torch.randn(2, 128, generator=torch.Generator().manual_seed(24)) * 0.5
    xs = dict(x)
    xs["k_tok"] = (x["k_tok"].float() + c).to(torch.bfloat16)
    xs["k_cart"] = x["k_cart"] + c
    g = _dev(xs)
    say("key shift")
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"])
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], o, lse,
                       g["dout"])
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, _ = O.attn_fwd(*args)
    gr = O.attn_bwd(*args, f64(x["dout"]), frozen_rows=1)
    assert rel(f64(o), o_ref) <= TOL_BF16
    for t in (0, 2, 4):                     # dQ, dV_tok, dV_cart: unchanged by the shift
        assert rel(f64(grads[t])[1:] if t == 4 else f64(grads[t]),
                   gr[t][1:] if t == 4 else gr[t]) <= TOL_BF16, t
    # dK (token and cartridge) too, up to bf16 rounding of the shifted keys
    assert rel(f64(grads[1]), gr[1]) <= TOL_BF16
    assert rel(f64(grads[3])[1:], gr[3][1:]) <= TOL_BF16


# ------------------------------------------------------------------ serving

def _make_cache(C, di, n_seqs, Hkv, d):
    bt = di.page_perm[: n_seqs * di.max_pages_per_seq].view(n_seqs, di.max_pages_per_seq)
    return C.PagedCache(n_seqs, Hkv, d, di.max_pages_per_seq, di.n_pages, bt, "cuda"), bt


def _gather_rows(cache, bt, s, L, d):
    """Rows 0..L-1 of sequence s read back from the pages: [L, Hkv, d]."""
    P = 16
    pages = bt[s, : (L + P - 1) // P].long().cuda()
    k = cache.k_pages[pages].permute(0, 2, 1, 3).reshape(-1, cache.n_kv_heads, d)[:L]
    v = cache.v_pages[pages].permute(0, 2, 1, 3).reshape(-1, cache.n_kv_heads, d)[:L]
    return k, v


def _serving_check(C, shape, n_seqs, p, max_gen):
    di = W.decode_inputs(shape, n_seqs=n_seqs, p=p, max_generated=max_gen)
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    cache, bt = _make_cache(C, di, n_seqs, Hkv, d)
    kc, vc = di.k_cart.cuda(), di.v_cart.cuda()
    oc = O.DenseCache(n_seqs, Hkv, d)
    say(shape.name, "write + append", n_seqs, p)
    for s in range(n_seqs):
        cache.write(s, kc, vc)
        assert cache.seq_len(s) == p
        oc.write(s, f64(di.k_cart), f64(di.v_cart))
        if di.generated[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    torch.cuda.synchronize()
    # the written prefix is bit-exact bf16 RNE of the f32 rows
    for s in (0, n_seqs - 1):
        k, v = _gather_rows(cache, bt, s, p, d)
        assert np.array_equal(f64(k), O.round_bf16(di.k_cart.numpy()))
        assert np.array_equal(f64(v), O.round_bf16(di.v_cart.numpy()))
    ws = C.workspace(cache.decode_workspace_size(Hq), "cuda")
    out = torch.empty(n_seqs, Hq, d, dtype=torch.bfloat16, device="cuda")
    say(shape.name, "decode attend-only")
    cache.decode(di.q.cuda(), out, ws)
    torch.cuda.synchronize()
    ref = O.decode_step(oc, f64(di.q))
    assert rel(f64(out), ref) <= TOL_BF16
    return cache, oc, di, ws, out


def test_serving_small_with_append(C):
    shape = W.DecodeShape("dec-small", 5, 40, 50, 8, 2, 128, 16, 13)
    cache, oc, di, ws, out = _serving_check(C, shape, 5, 40, 50)
    # one more step that appends a new token first (it sees itself)
    g = torch.Generator().manual_seed(99)
    kn = torch.randn(5, 2, 128, generator=g).to(torch.bfloat16)
    vn = torch.randn(5, 2, 128, generator=g).to(torch.bfloat16)
    qn = torch.randn(5, 8, 128, generator=g).to(torch.bfloat16)
    lens = [cache.seq_len(s) for s in range(5)]
    say("decode with append")
    cache.decode(qn.cuda(), out, ws, k_new=kn.cuda(), v_new=vn.cuda())
    torch.cuda.synchronize()
    assert [cache.seq_len(s) for s in range(5)] == [l + 1 for l in lens]
    assert f64(cache.seq_lens).astype(int).tolist() == [l + 1 for l in lens]
    ref = O.decode_step(oc, f64(qn), f64(kn), f64(vn))
    assert rel(f64(out), ref) <= TOL_BF16
    # writing into a sequence that already holds rows is refused
    with pytest.raises(C.CartError) as e:
        cache.write(0, di.k_cart.cuda(), di.v_cart.cuda())
    assert e.value.status == C.CART_ERR_CACHE_NOT_EMPTY
    cache.reset(0)
    assert cache.seq_len(0) == 0


def test_serving_parity_decode_equals_fwd(C):
    """Decode behind the written prefix, token by token at positions p, p+1,
    ..., equals the GPU forward of the same tokens behind the same cartridge
    with bf16-rounded rows (serving parity)."""
    p, n, Hq, Hkv, d = 64, 24, 8, 2, 128
    sh = _shape("sp", 1, n, p, Hq, Hkv, d, torch.bfloat16, torch.float32, 31)
    x = _dev(W.train_inputs(sh))
    q, kt = x["q"].clone(), x["k_tok"].clone()
    C.cart_rope_tokens(q, kt, pos_base=p, theta=TH)
    kc_b = x["k_cart"].to(torch.bfloat16)
    vc_b = x["v_cart"].to(torch.bfloat16)
    say("serving parity fwd")
    o_fwd, _ = C.attn_fwd(q, kt, x["v_tok"], kc_b, vc_b)
    bt = torch.arange(8, dtype=torch.int32).view(1, 8)
    cache = C.PagedCache(1, Hkv, d, 8, 8, bt, "cuda")
    cache.write(0, x["k_cart"], x["v_cart"])
    ws = C.workspace(cache.decode_workspace_size(Hq), "cuda")
    out = torch.empty(1, Hq, d, dtype=torch.bfloat16, device="cuda")
    outs = []
    for t in range(n):
        say("decode step", t)
        qq = x["q"][:, t].clone()                       # [1, Hq, d] raw
        kk = x["k_tok"][:, t].clone()
        # rotate at the cache's length (the new token's position)
        C.cart_rope_tokens(qq[:, None], kk[:, None], pos_base=0, pos_offsets=cache.seq_lens,
                           theta=TH)
        cache.decode(qq, out, ws, k_new=kk, v_new=x["v_tok"][:, t].contiguous())
        outs.append(out.clone())
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, 1)
    assert rel(f64(o_dec), f64(o_fwd)) <= TOL_BF16


def test_config_serving_decode(C):
    sh = W.DECODE
    _serving_check(C, sh, sh.n_seqs, sh.p, sh.max_generated)


# GQA groups 1, 2, 4, 8 at head_dim 64 and 128, with sequences of very
# different lengths in one cache: 1 row, a few pages, a mid length and the
# full capacity, so that some sequences have fewer splits than the launch's
# maximum (idle splits, whose partials weigh nothing). At 40 pages per
# sequence (5 splits) the splits are the waves of one workgroup, merged on
# chip (three of its 8 waves always idle); at 80 (10 splits) one workgroup
# per split, merged by the second kernel; 16 and 24 pages give workgroups of
# 2 and 4 waves (2 and 3 splits).
DECODE_VARIANTS = [(g, d, mp) for mp in (40, 80) for d in (64, 128) for g in (1, 2, 4, 8)]
DECODE_VARIANTS += [(4, 128, 16), (8, 64, 16), (2, 128, 24), (4, 64, 24)]
WAVES_OF_PAGES = {16: 2, 24: 4, 40: 8, 80: 0}


@pytest.mark.parametrize("g,d,max_pages", DECODE_VARIANTS,
                         ids=[f"g{g}-d{d}-mp{mp}" for g, d, mp in DECODE_VARIANTS])
def test_decode_variants_ragged(C, g, d, max_pages):
    Hkv = 2
    Hq = g * Hkv
    full = 16 * max_pages                            # rows per sequence at capacity
    prefix = [1, 20, min(257, full // 2), full - 40, 100]
    gen = [0, 13, 50, 40, 0]
    di = W.decode_inputs_ragged(prefix, gen, Hq, Hkv, d, max_pages, seed=300 + 10 * g + d)
    n_seqs = len(prefix)
    cache = C.PagedCache(n_seqs, Hkv, d, max_pages, di.n_pages,
                         di.page_perm.view(n_seqs, max_pages), "cuda")
    oc = O.DenseCache(n_seqs, Hkv, d)
    say("decode variant", g, d)
    for s in range(n_seqs):
        cache.write(s, di.k_cart[s].cuda(), di.v_cart[s].cuda())
        oc.write(s, f64(di.k_cart[s]), f64(di.v_cart[s]))
        if gen[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    lens = [cache.seq_len(s) for s in range(n_seqs)]
    assert lens == [a + b for a, b in zip(prefix, gen)] and max(lens) == full
    sc = cache.decode_schedule(Hq)
    # at least 2 splits for the longest sequence: the merge really merges
    assert sc.max_splits == max_pages // 8 >= 2
    assert sc.waves_per_group == WAVES_OF_PAGES[max_pages]
    nbytes = cache.decode_workspace_size(Hq)
    ws = C.workspace(nbytes, "cuda")
    out = torch.empty(n_seqs, Hq, d, dtype=torch.bfloat16, device="cuda")
    cache.decode(di.q.cuda(), out, ws)
    torch.cuda.synchronize()
    assert rel(f64(out), O.decode_step(oc, f64(di.q))) <= TOL_BF16
    # then a step that appends one row to every sequence: the full one is
    # first reset and given its prefix alone again (in the oracle too)
    cache.reset(3)
    cache.write(3, di.k_cart[3].cuda(), di.v_cart[3].cuda())
    oc.k[3], oc.v[3] = oc.k[3][:prefix[3]], oc.v[3][:prefix[3]]
    cache.decode(di.q.cuda(), out, ws, k_new=di.k_new.cuda(), v_new=di.v_new.cuda())
    torch.cuda.synchronize()
    ref = O.decode_step(oc, f64(di.q), f64(di.k_new), f64(di.v_new))
    assert rel(f64(out), ref) <= TOL_BF16
    cache.close()


@pytest.mark.parametrize("mode", ["f32", "bf16-f32rows"])
def test_custom_softmax_scale(C, mode):
    """A positive scale other than 1/sqrt(d) reaches every kernel: forward,
    both backward kernels and the decode (compared with the oracle at the
    same scale)."""
    tok = torch.float32 if mode == "f32" else torch.bfloat16
    name, B, n, p, Hq, Hkv, d = ("scale", 2, 90, 150, 8, 2, 128)
    sc = 0.05
    x = W.train_inputs(_shape(name, B, n, p, Hq, Hkv, d, tok, torch.float32, 78))
    g = _dev(x)
    say("custom scale", mode)
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], scale=sc)
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], g["k_cart"], g["v_cart"], o, lse,
                       g["dout"], scale=sc)
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, _ = O.attn_fwd(*args, scale=sc)
    gr = O.attn_bwd(*args, f64(x["dout"]), scale=sc, frozen_rows=1)
    got = dict(o=o, dq=grads[0], dk_tok=grads[1], dv_tok=grads[2], dk_cart=grads[3],
               dv_cart=grads[4])
    ref = dict(o=o_ref, dq=gr[0], dk_tok=gr[1], dv_tok=gr[2], dk_cart=gr[3], dv_cart=gr[4])
    _compare(got, ref, TOL_F32 if mode == "f32" else TOL_BF16, 1, names=list(ref))


def test_custom_scale_decode(C):
    shape = W.DecodeShape("dec-scale", 3, 40, 30, 8, 2, 128, 16, 14)
    di = W.decode_inputs(shape, n_seqs=3, p=40, max_generated=30)
    cache, bt = _make_cache(C, di, 3, 2, 128)
    oc = O.DenseCache(3, 2, 128)
    for s in range(3):
        cache.write(s, di.k_cart.cuda(), di.v_cart.cuda())
        oc.write(s, f64(di.k_cart), f64(di.v_cart))
        if di.generated[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    out = torch.empty(3, 8, 128, dtype=torch.bfloat16, device="cuda")
    say("custom scale decode")
    cache.decode(di.q.cuda(), out, C.workspace(cache.decode_workspace_size(8), "cuda"), scale=0.3)
    torch.cuda.synchronize()
    assert rel(f64(out), O.decode_step(oc, f64(di.q), scale=0.3)) <= TOL_BF16
