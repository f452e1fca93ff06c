"""Seeded sweeps of random small geometries, GPU (through the C ABI) against
the oracles: attention forward and backward, and the decode / verify step.

The hand-picked parity cases pin the edges one by one; these sweeps draw
the geometry itself (batch, queries, cartridge length, frozen rows, GQA
group, head_dim, sliding window, row dtype; for the cache, sequence lengths,
page capacity, GQA group, draft count) from a fixed seed, so that
combinations nobody picked are checked too. Tolerances as in the other
parity tests: 2e-2 normwise for bf16 inputs, 1e-5 in the float32 mode;
frozen rows and rows no query sees must be exactly zero.

Pages: "Cartridges: trained KV-prefix corpus compression", sections
"Semantics (pinned to the reference implementation)" (the forward, the
backward through the concat, the frozen sink, serving behind the written
prefix) and "gemma4 (measured)" (a window that can cut through the prefix).
"""

import numpy as np
import pytest
import torch

from oracle import cartattn_oracle as O
from oracle import variants as V
from long_context_kv_amd import workloads as W
from tests._common import f64, rel, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_kv_amd import cartattn
    return cartattn


def _attention_cases(n_cases=24, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        b = int(rng.integers(1, 4))
        n = int(rng.integers(1, 300))
        p = int([0, rng.integers(1, 64), rng.integers(64, 700)][rng.integers(0, 3)])
        f = int(rng.integers(0, min(p, 3) + 1))
        window = int([0, 0, rng.integers(1, p + n + 40)][rng.integers(0, 3)])
        mode = str(rng.choice(["bf16-f32rows", "bf16-bf16rows", "bf16-f32rows", "f32"]))
        cases.append((i, b, n, p, f, g * hkv, hkv, d, window, mode))
    return cases


ATTN = _attention_cases()


def _err(gpu, ref):
    """Normwise error; a reference that is zero in exact arithmetic (a
    one-row window makes dQ and dK vanish) is compared in absolute terms."""
    if float(np.max(np.abs(ref))) > 1e-6:
        return rel(gpu, ref)
    return float(np.max(np.abs(gpu)))


@pytest.mark.parametrize("case", ATTN, ids=[
    f"a{c[0]}-B{c[1]}-n{c[2]}-p{c[3]}-f{c[4]}-hq{c[5]}-hkv{c[6]}-d{c[7]}-w{c[8]}-{c[9]}"
    for c in ATTN])
def test_attention_sweep(C, case):
    i, B, n, p, f, Hq, Hkv, d, window, mode = case
    tok = torch.float32 if mode == "f32" else torch.bfloat16
    row = torch.bfloat16 if mode == "bf16-bf16rows" else torch.float32
    say("sweep attention", case)
    x = W.train_inputs(W.TrainShape(f"sweep{i}", B, n, p, Hq, Hkv, d, tok, row, 900 + i))
    g = {k: v.cuda().contiguous() for k, v in x.items()}
    kc = g["k_cart"] if p else None
    vc = g["v_cart"] if p else None
    o, lse = C.attn_fwd(g["q"], g["k_tok"], g["v_tok"], kc, vc, frozen_rows=f, window=window)
    grads = C.attn_bwd(g["q"], g["k_tok"], g["v_tok"], kc, vc, o, lse, g["dout"],
                       frozen_rows=f, window=window)
    torch.cuda.synchronize()
    args = [f64(x[k]) for k in ("q", "k_tok", "v_tok", "k_cart", "v_cart")]
    o_ref, lse_ref = V.attn_fwd_window(*args, window)
    ref = V.attn_bwd_window(*args, f64(x["dout"]), window, frozen_rows=f)
    tol = TOL_F32 if mode == "f32" else TOL_BF16
    errs = {"o": rel(f64(o), o_ref)}
    for name, gpu, r in zip(("dq", "dk_tok", "dv_tok"), grads[:3], ref[:3]):
        errs[name] = _err(f64(gpu), r)
    if p:
        # rows below the frozen count, and rows no query sees, are exactly 0
        first_seen = max(0, p - window + 1) if window else 0
        for name, gpu, r in zip(("dk_cart", "dv_cart"), grads[3:], ref[3:]):
            gg = f64(gpu)
            assert np.all(gg[:max(f, first_seen)] == 0), name
            if p > f:
                errs[name] = _err(gg[f:], r[f:])
    # a query that sees no row at all (not possible: it always sees itself)
    assert np.all(np.isfinite(f64(lse)))
    assert np.max(np.abs(f64(lse) - lse_ref)) <= (1e-5 if mode == "f32" else 2e-2)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, errs


# Decode / verify: the page capacity is chosen so that the splits per
# sequence at full capacity cycle through 1, 2, 3, 5, 8, 9 and 20 (8 pages
# per split while the cache is small), i.e. workgroups of 1, 2, 4 and 8 waves
# merged on chip and one-wave workgroups merged by the second kernel.
SPLIT_TARGETS = [1, 2, 3, 5, 8, 9, 20]


def _decode_cases(n_cases=14, seed=4711):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        ms = SPLIT_TARGETS[i % len(SPLIT_TARGETS)]
        mp = 8 * ms - int(rng.integers(0, 4))            # pages per sequence
        S = int(rng.integers(1, 7))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        k = int(rng.choice([1, 1, 2, 3, 5, 8]))          # 1: decode, more: verify
        cap = 16 * mp
        lens = [int(rng.integers(1, cap - k + 1)) for _ in range(S)]
        lens[int(rng.integers(0, S))] = cap - k              # one sequence filled up
        cases.append((i, S, hkv, g * hkv, d, mp, k, lens))
    return cases


DEC = _decode_cases()


@pytest.mark.parametrize("case", DEC, ids=[
    f"d{c[0]}-S{c[1]}-hkv{c[2]}-hq{c[3]}-d{c[4]}-mp{c[5]}-k{c[6]}" for c in DEC])
def test_decode_sweep(C, case):
    i, S, Hkv, Hq, d, mp, k, lens = case
    say("sweep decode", case)
    prefix = [max(1, L // 2) for L in lens]
    gen = [L - P for L, P in zip(lens, prefix)]
    di = W.decode_inputs_ragged(prefix, gen, Hq, Hkv, d, mp, seed=1300 + i)
    cache = C.PagedCache(S, Hkv, d, mp, di.n_pages, di.page_perm.view(S, mp), "cuda")
    oc = O.DenseCache(S, Hkv, d)
    for s in range(S):
        cache.write(s, di.k_cart[s].cuda(), di.v_cart[s].cuda())
        oc.write(s, f64(di.k_cart[s]), f64(di.v_cart[s]))
        if gen[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    assert [cache.seq_len(s) for s in range(S)] == lens
    sc = cache.decode_schedule(Hq, k)
    waves = 1
    while waves < sc.max_splits:
        waves *= 2
    assert sc.waves_per_group == (waves if sc.max_splits <= 8 else 0)
    ws = C.workspace(sc.workspace_bytes, "cuda")
    rg = torch.Generator().manual_seed(1400 + i)
    if k == 1:
        kn = torch.randn(S, Hkv, d, generator=rg).to(torch.bfloat16)
        vn = torch.randn(S, Hkv, d, generator=rg).to(torch.bfloat16)
        q = torch.randn(S, Hq, d, generator=rg).to(torch.bfloat16)
        out = torch.empty(S, Hq, d, dtype=torch.bfloat16, device="cuda")
        cache.decode(q.cuda(), out, ws, k_new=kn.cuda(), v_new=vn.cuda())
        torch.cuda.synchronize()
        ref = O.decode_step(oc, f64(q), f64(kn), f64(vn))
    else:
        kn = torch.randn(S, k, Hkv, d, generator=rg).to(torch.bfloat16)
        vn = torch.randn(S, k, Hkv, d, generator=rg).to(torch.bfloat16)
        q = torch.randn(S, k, Hq, d, generator=rg).to(torch.bfloat16)
        out = torch.empty(S, k, Hq, d, dtype=torch.bfloat16, device="cuda")
        cache.verify(q.cuda(), kn.cuda(), vn.cuda(), out, ws)
        torch.cuda.synchronize()
        ref = V.verify_step(oc, f64(q), f64(kn), f64(vn))
    assert [cache.seq_len(s) for s in range(S)] == [L + k for L in lens]
    assert rel(f64(out), ref) <= TOL_BF16
    cache.close()


def test_decode_sweep_covers_every_merge_path():
    """Host-side check of the sweep itself: its geometries reach every
    workgroup size of the on-chip merge and the merge kernel."""
    got = set()
    for (_, S, Hkv, Hq, d, mp, k, _lens) in DEC:
        ms = -(-mp // 8)
        w = 1
        while w < ms:
            w *= 2
        got.add(w if ms <= 8 else 0)
    assert got == {0, 1, 2, 4, 8}
