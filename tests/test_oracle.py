"""Pins of the CPU float64 oracle against things other than itself.

Each test checks the oracle against what the pages and the mathematics fix:
the zero-training prefill-equivalence gate, finite differences, the frozen
sink row, a library routine (torch CPU float64 attention + autograd), closed
forms of softmax attention, RoPE identities with hand-computed values, and
torch's bfloat16 cast. The pages print no worked-example values, so no pin
is a printed number (see tests/golden/README.md).

Pages: "Cartridges: trained KV-prefix corpus compression", sections
"Semantics (pinned to the reference implementation)" and "Evidence";
"RIG minimal cognition engine implementation hand-off", section 5 (RoPE
warning).
"""

import re

import numpy as np
import pytest
import torch

from oracle import cartattn_oracle as O
from long_context_kv_amd import workloads as W

TH = W.THETA


def _np(t):
    return t.double().numpy()


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _tiny(seed=1, B=1, n=16, p=8, Hq=4, Hkv=2, d=64):
    shape = W.TrainShape("t", B, n, p, Hq, Hkv, d, torch.float32, torch.float32, seed)
    x = W.train_inputs(shape)
    return {k: _np(v) for k, v in x.items()}


def _prefill_setup(B=1, p=8, n=16, Hq=4, Hkv=2, d=64, seed=101):
    """Raw rows of T = p + n positions; the cartridge is the rotated first p
    rows (the model's own K/V), tokens are raw rows p.. rotated at p + i."""
    q, k, v, dout = W.prefill_raw(p + n, Hq, Hkv, d, seed, batch=B)
    q, k, v, dout = _np(q), _np(k), _np(v), _np(dout)
    # one shared prefix: every sequence starts with batch 0's first p rows
    q[:, :p] = q[0:1, :p]
    k[:, :p] = k[0:1, :p]
    v[:, :p] = v[0:1, :p]
    T = p + n
    pos_all = O.token_positions(B, T, 0)
    qr = O.rope(q, pos_all, TH)
    kr = O.rope(k, pos_all, TH)
    k_cart = kr[0, :p]
    v_cart = v[0, :p]
    pos_tok = O.token_positions(B, n, p)
    q_tok = O.rope(q[:, p:], pos_tok, TH)
    k_tok = O.rope(k[:, p:], pos_tok, TH)
    return dict(qr=qr, kr=kr, v=v, dout=dout, q_tok=q_tok, k_tok=k_tok,
                v_tok=v[:, p:], k_cart=k_cart, v_cart=v_cart, p=p)


# ---------------------------------------------------------------- prefill gate

@pytest.mark.parametrize("B,p,n,Hq,Hkv,d", [(1, 8, 16, 4, 2, 64), (2, 5, 11, 6, 2, 32),
                                            (1, 1, 3, 2, 2, 16)])
def test_prefill_equivalence_forward(B, p, n, Hq, Hkv, d):
    s = _prefill_setup(B, p, n, Hq, Hkv, d)
    o_c, lse_c = O.attn_fwd(s["q_tok"], s["k_tok"], s["v_tok"], s["k_cart"], s["v_cart"])
    o_ref, lse_ref = O.causal_prefill(s["qr"], s["kr"], s["v"])
    assert _rel(o_c, o_ref[:, p:]) <= 1e-12
    assert np.max(np.abs(lse_c - lse_ref[:, :, p:])) <= 1e-12


def test_prefill_equivalence_gradients():
    """With dO = 0 on the first p rows, the real prefill's gradients equal the
    cartridge path's: queries < p then carry no gradient."""
    p = 8
    s = _prefill_setup(B=1, p=p)
    dout = s["dout"].copy()
    dout[:, :p] = 0.0
    dq_r, dk_r, dv_r = O.causal_prefill_bwd(s["qr"], s["kr"], s["v"], dout)
    dq, dkt, dvt, dkc, dvc = O.attn_bwd(s["q_tok"], s["k_tok"], s["v_tok"], s["k_cart"],
                                        s["v_cart"], dout[:, p:], frozen_rows=1)
    assert _rel(dq, dq_r[:, p:]) <= 1e-12
    assert _rel(dkt, dk_r[:, p:]) <= 1e-12
    assert _rel(dvt, dv_r[:, p:]) <= 1e-12
    assert _rel(dkc[1:], dk_r[0, 1:p]) <= 1e-12
    assert _rel(dvc[1:], dv_r[0, 1:p]) <= 1e-12
    assert np.all(dkc[0] == 0.0) and np.all(dvc[0] == 0.0)


def test_shifted_base_position_breaks_equivalence():
    """A cartridge mounted with tokens at p+1.. instead of p.. does not
    reproduce the prefill (the RoPE warning of the RIG hand-off, section 5)."""
    p, n = 8, 16
    s = _prefill_setup(B=1, p=p, n=n)
    q, k, v, _ = W.prefill_raw(p + n, 4, 2, 64, 101)
    q, k = _np(q), _np(k)
    bad = O.token_positions(1, n, p + 1)
    o_bad, _ = O.attn_fwd(O.rope(q[:, p:], bad, TH), O.rope(k[:, p:], bad, TH), s["v_tok"],
                          s["k_cart"], s["v_cart"])
    o_ref, _ = O.causal_prefill(s["qr"], s["kr"], s["v"])
    assert _rel(o_bad, o_ref[:, p:]) > 1e-3


# ---------------------------------------------------------- finite differences

def test_finite_difference_gradients():
    """Central differences of sum(O * dO) through concat + attention into the
    trainable rows, kv_seq > q_seq, GQA (the "Evidence" gradcheck)."""
    x = _tiny(seed=7)
    names = ["q", "k_tok", "v_tok", "k_cart", "v_cart"]
    grads = O.attn_bwd(x["q"], x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"],
                       x["dout"], frozen_rows=1)
    rng = np.random.default_rng(0)
    for t, name in enumerate(names):
        def loss(val, name=name):
            args = dict(x)
            args[name] = val
            o, _ = O.attn_fwd(args["q"], args["k_tok"], args["v_tok"], args["k_cart"],
                              args["v_cart"])
            return float(np.sum(o * x["dout"]))
        size = x[name].size
        idx = list(rng.choice(size, size=min(size, 48), replace=False))
        if name in ("k_cart", "v_cart"):
            row = x[name][0].size
            idx = [i for i in idx if i >= row]        # trainable rows only
        fd = O.fd_grad(loss, x[name], idx)
        an = grads[t].reshape(-1)[idx]
        err = np.max(np.abs(fd - an)) / np.max(np.abs(an))
        assert err <= 1e-7, (name, err)


def test_frozen_row_zero_and_observable():
    """Rows below frozen_rows get exactly zero gradient, while the gradient
    they would receive unfrozen is non-zero (so the freeze is observable)."""
    x = _tiny(seed=3)
    args = (x["q"], x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"], x["dout"])
    g1 = O.attn_bwd(*args, frozen_rows=1)
    g0 = O.attn_bwd(*args, frozen_rows=0)
    g3 = O.attn_bwd(*args, frozen_rows=3)
    for dc1, dc0, dc3 in zip(g1[3:], g0[3:], g3[3:]):
        assert np.all(dc1[0] == 0.0)
        assert np.all(dc3[:3] == 0.0)
        assert np.max(np.abs(dc0[0])) > 1e-3
        assert np.array_equal(dc1[1:], dc0[1:])
        assert np.array_equal(dc3[3:], dc0[3:])
    for a, b in zip(g1[:3], g0[:3]):
        assert np.array_equal(a, b)


# ------------------------------------------------------------ library routine

def _torch_reference(x, frozen_rows, scale=None):
    """torch CPU float64 scaled_dot_product_attention with an explicit
    boolean mask and repeat_interleave for GQA, differentiated by autograd."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in x.items()
         if k != "dout"}
    B, n, Hq, d = t["q"].shape
    p, Hkv = t["k_cart"].shape[0], t["k_tok"].shape[2]
    g = Hq // Hkv
    K = torch.cat([t["k_cart"].unsqueeze(0).expand(B, p, Hkv, d), t["k_tok"]], dim=1)
    V = torch.cat([t["v_cart"].unsqueeze(0).expand(B, p, Hkv, d), t["v_tok"]], dim=1)
    K = K.repeat_interleave(g, dim=2).transpose(1, 2)
    V = V.repeat_interleave(g, dim=2).transpose(1, 2)
    Q = t["q"].transpose(1, 2)
    i = torch.arange(n)[:, None]
    j = torch.arange(p + n)[None, :]
    mask = j <= i + p
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                           scale=scale)
    out = out.transpose(1, 2)
    (out * torch.tensor(x["dout"])).sum().backward()
    return out.detach().numpy(), [t[k].grad.numpy() for k in
                                  ("q", "k_tok", "v_tok", "k_cart", "v_cart")]


@pytest.mark.parametrize("B,n,p,Hq,Hkv,d,scale", [(1, 16, 8, 4, 2, 64, None),
                                                  (3, 13, 21, 8, 2, 32, 0.3),
                                                  (2, 9, 0, 4, 4, 16, None)])
def test_against_torch_sdpa_autograd(B, n, p, Hq, Hkv, d, scale):
    x = _tiny(seed=11, B=B, n=n, p=p, Hq=Hq, Hkv=Hkv, d=d)
    f = 1 if p > 0 else 0
    o_ref, g_ref = _torch_reference(x, f, scale)
    o, _ = O.attn_fwd(x["q"], x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"],
                      scale or 0.0)
    assert _rel(o, o_ref) <= 1e-12
    g = O.attn_bwd(x["q"], x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"], x["dout"],
                   scale or 0.0, frozen_rows=f)
    for t in range(3):
        assert _rel(g[t], g_ref[t]) <= 1e-12
    for t in (3, 4):
        if p > f:
            assert _rel(g[t][f:], g_ref[t][f:]) <= 1e-12
        assert np.all(g[t][:f] == 0.0)


# ---------------------------------------------------------------- closed forms

def test_closed_form_uniform_scores():
    """All-zero queries make every visible score equal, so O is the plain
    mean of the visible value rows and LSE = log(#visible) (worked by hand:
    query i of a p-row cartridge sees p + i + 1 rows)."""
    x = _tiny(seed=5)
    q = np.zeros_like(x["q"])
    o, lse = O.attn_fwd(q, x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"])
    p, n = x["k_cart"].shape[0], q.shape[1]
    for i in range(n):
        for h in range(q.shape[2]):
            kv = h // 2
            rows = np.concatenate([x["v_cart"][:, kv], x["v_tok"][0, :i + 1, kv]], 0)
            assert np.max(np.abs(o[0, i, h] - rows.mean(0))) <= 1e-13
            assert abs(lse[0, h, i] - np.log(p + i + 1)) <= 1e-13


def test_closed_form_two_keys():
    """One query, p = 1, n = 1, d = 2: scores s0 = q.k0 / sqrt(2) and
    s1 = q.k1 / sqrt(2), so O = (e^s0 v0 + e^s1 v1) / (e^s0 + e^s1)."""
    q = np.array([[[[1.0, 2.0]]]])
    kc = np.array([[[0.5, -1.0]]])
    kt = np.array([[[[2.0, 1.0]]]])
    vc = np.array([[[3.0, -2.0]]])
    vt = np.array([[[[-1.0, 4.0]]]])
    s0 = (1.0 * 0.5 + 2.0 * -1.0) / np.sqrt(2.0)
    s1 = (1.0 * 2.0 + 2.0 * 1.0) / np.sqrt(2.0)
    w0, w1 = np.exp(s0), np.exp(s1)
    expect = (w0 * vc[0, 0] + w1 * vt[0, 0, 0]) / (w0 + w1)
    o, lse = O.attn_fwd(q, kt, vt, kc, vc)
    assert np.max(np.abs(o[0, 0, 0] - expect)) <= 1e-14
    assert abs(lse[0, 0, 0] - np.log(w0 + w1)) <= 1e-14


def test_invariants():
    """Sum_j dV_j = Sum of dO over the group; Sum_j dK_j = 0 (rows of dS sum
    to zero); adding a vector to every key leaves O unchanged; constant V
    rows give that constant."""
    x = _tiny(seed=9, B=2, n=12, p=6, Hq=6, Hkv=3, d=32)
    dq, dkt, dvt, dkc, dvc = O.attn_bwd(x["q"], x["k_tok"], x["v_tok"], x["k_cart"],
                                        x["v_cart"], x["dout"], frozen_rows=0)
    g = 2
    for kv in range(3):
        sdv = dvc[:, kv].sum(0) + dvt[:, :, kv].sum((0, 1))
        sdo = x["dout"][:, :, kv * g:(kv + 1) * g].sum((0, 1, 2))
        assert np.max(np.abs(sdv - sdo)) <= 1e-12
        sdk = dkc[:, kv].sum(0) + dkt[:, :, kv].sum((0, 1))
        assert np.max(np.abs(sdk)) <= 1e-12
    o, _ = O.attn_fwd(x["q"], x["k_tok"], x["v_tok"], x["k_cart"], x["v_cart"])
    c = np.random.default_rng(1).standard_normal((3, 32))
    o2, _ = O.attn_fwd(x["q"], x["k_tok"] + c, x["v_tok"], x["k_cart"] + c, x["v_cart"])
    assert _rel(o2, o) <= 1e-12
    const = np.random.default_rng(2).standard_normal((3, 32))
    vt = np.broadcast_to(const, x["v_tok"].shape)
    vc = np.broadcast_to(const, x["v_cart"].shape)
    o3, _ = O.attn_fwd(x["q"], x["k_tok"], vt, x["k_cart"], vc)
    for h in range(6):
        assert np.max(np.abs(o3[:, :, h] - const[h // 2])) <= 1e-12


# ----------------------------------------------------------------------- RoPE

def test_rope_hand_values():
    """Hand-computed angles: k = 0 has frequency theta**0 = 1, so position 1
    turns the first pair by exactly 1 rad; with d = 4 and theta = 1e6 the
    second pair has frequency 1e6**(-1/2) = 1e-3, so position 1000 turns it
    by exactly 1 rad as well."""
    x = np.array([[[[0.3, -0.7, 1.1, 0.4]]]])
    c, s = np.cos(1.0), np.sin(1.0)
    r = O.rope(x, np.array([[1]]), 1e6)
    assert abs(r[0, 0, 0, 0] - (0.3 * c - 1.1 * s)) <= 1e-15
    assert abs(r[0, 0, 0, 2] - (1.1 * c + 0.3 * s)) <= 1e-15
    r = O.rope(x, np.array([[1000]]), 1e6)
    assert abs(r[0, 0, 0, 1] - (-0.7 * c - 0.4 * s)) <= 1e-14
    assert abs(r[0, 0, 0, 3] - (0.4 * c + -0.7 * s)) <= 1e-14


def test_rope_identities():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 10, 3, 64))
    y = rng.standard_normal((2, 10, 3, 64))
    pos = O.token_positions(2, 10, 37, [0, 5])
    # position 0 is the identity
    assert np.array_equal(O.rope(x, np.zeros((2, 10), int), TH), x)
    # inverse undoes forward; norms are preserved
    r = O.rope(x, pos, TH)
    assert np.max(np.abs(O.rope(r, pos, TH, inverse=True) - x)) <= 1e-13
    assert np.max(np.abs(np.linalg.norm(r, axis=-1) - np.linalg.norm(x, axis=-1))) <= 1e-12
    # <R(m) a, R(n) b> depends only on n - m
    a, b = x[0, 0, 0][None, None, None], y[0, 0, 0][None, None, None]
    d1 = np.sum(O.rope(a, np.array([[3]]), TH) * O.rope(b, np.array([[10]]), TH))
    d2 = np.sum(O.rope(a, np.array([[103]]), TH) * O.rope(b, np.array([[110]]), TH))
    assert abs(d1 - d2) <= 1e-12
    # inverse is the adjoint: <R a, b> = <a, R^T b>
    lhs = np.sum(O.rope(x, pos, TH) * y)
    rhs = np.sum(x * O.rope(y, pos, TH, inverse=True))
    assert abs(lhs - rhs) <= 1e-11
    # rotating T rows at base 0 and slicing [p:] = rotating those rows at base p
    p = 7
    full = O.rope(x, O.token_positions(2, 10, 0), TH)
    part = O.rope(x[:, p:], O.token_positions(2, 10 - p, p), TH)
    assert np.array_equal(full[:, p:], part)


# ---------------------------------------------------------------- bf16 + cache

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(6)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),      # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38], np.float32),
    ])
    # exact ties: low 16 bits 0x8000, both parities of the kept bit
    u = rng.integers(0, 2 ** 31, 4000, dtype=np.uint64)
    ties = ((u & ~np.uint64(0xFFFF)) | np.uint64(0x8000)).astype(np.uint32).view(np.float32)
    vals = np.concatenate([vals, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    got = O.round_bf16(vals).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.round_bf16(np.array([np.nan], np.float32)))[0]


def test_cache_write_rules():
    c = O.DenseCache(2, 2, 8)
    kc = np.random.default_rng(0).standard_normal((5, 2, 8)).astype(np.float32)
    c.write(0, kc, kc)
    assert c.seq_len(0) == 5 and c.seq_len(1) == 0
    assert np.array_equal(c.k[0], O.round_bf16(kc))
    with pytest.raises(ValueError):
        c.write(0, kc, kc)


def test_serving_parity_decode_equals_cartridge_forward():
    """Decode behind the written prefix, one token at a time at positions
    p, p+1, ..., equals the cartridge forward over the same bf16-rounded
    rows (the "Evidence" serving-parity check, and the RIG hand-off's
    restored-state decode == full-context decode)."""
    p, n, Hq, Hkv, d = 8, 6, 4, 2, 32
    x = _tiny(seed=21, B=1, n=n, p=p, Hq=Hq, Hkv=Hkv, d=d)
    pos = O.token_positions(1, n, p)
    q = O.rope(x["q"], pos, TH)
    k = O.rope(x["k_tok"], pos, TH)
    cache = O.DenseCache(1, Hkv, d)
    cache.write(0, x["k_cart"], x["v_cart"])
    outs = []
    for t in range(n):
        assert cache.seq_len(0) == p + t          # new token's position
        outs.append(O.decode_step(cache, q[:, t], k[:, t], x["v_tok"][:, t]))
    o_dec = np.stack(outs, axis=1)
    rb = O.round_bf16
    o_ref, _ = O.attn_fwd(q, rb(k), rb(x["v_tok"]), rb(x["k_cart"]), rb(x["v_cart"]))
    assert _rel(o_dec, o_ref) <= 1e-12


def test_decode_attend_only_equals_fwd_q1():
    """Without a new row, decode over L stored rows equals the forward with
    q_seq = 1, cartridge = rows 0..L-2 and the last row as the token."""
    rng = np.random.default_rng(8)
    cache = O.DenseCache(3, 2, 16)
    for s in range(3):
        cache.append(s, rng.standard_normal((4 + s, 2, 16)), rng.standard_normal((4 + s, 2, 16)))
    q = rng.standard_normal((3, 6, 16))
    o = O.decode_step(cache, q)
    for s in range(3):
        K, V = cache.k[s], cache.v[s]
        ref, _ = O.attn_fwd(q[s][None, None], K[None, -1:], V[None, -1:], K[:-1], V[:-1])
        assert _rel(o[s], ref[0, 0]) <= 1e-12


def test_oracle_is_independent_of_the_hip_path():
    """The oracle imports only numpy; the HIP sources never mention it."""
    import pathlib
    root = pathlib.Path(__file__).resolve().parents[1]
    src = (root / "oracle" / "cartattn_oracle.py").read_text()
    imports = [l for l in src.splitlines() if l.startswith(("import ", "from "))]
    assert all(("numpy" in l) or ("__future__" in l) for l in imports), imports
    pat = re.compile(r"^\s*(from\s+oracle|import\s+oracle)|cartattn_oracle", re.M)
    for f in list((root / "long_context_kv_amd").rglob("*")) + list((root / "include").rglob("*")):
        if f.suffix in (".py", ".hip", ".cpp", ".h", ".hpp"):
            assert not pat.search(f.read_text()), f
