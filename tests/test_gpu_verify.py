"""GPU parity of the multi-token verify step behind the serving cache
(cart_decode_verify) and of the truncating rewind (cart_cache_truncate),
through the C ABI, against the oracle's verify step.

Page: "Cartridges: trained KV-prefix corpus compression", section "Batched
self-study (measured)": drafts verified per stream against its own cache,
greedy acceptance per row, truncating rewinds.
"""

import numpy as np
import pytest
import torch

from oracle import cartattn_oracle as O
from oracle import variants as V
from long_context_kv_amd import workloads as W
from tests._common import f64, rel, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def C():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_kv_amd import cartattn
    return cartattn


def _filled(C, prefix, gen, Hq, Hkv, d, mp, seed):
    di = W.decode_inputs_ragged(prefix, gen, Hq, Hkv, d, mp, seed=seed)
    n = len(prefix)
    cache = C.PagedCache(n, Hkv, d, mp, di.n_pages, di.page_perm.view(n, mp), "cuda")
    oc = O.DenseCache(n, Hkv, d)
    for s in range(n):
        cache.write(s, di.k_cart[s].cuda(), di.v_cart[s].cuda())
        oc.write(s, f64(di.k_cart[s]), f64(di.v_cart[s]))
        if gen[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    return cache, oc


def _drafts(S, k, Hq, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    return r(S, k, Hq, d), r(S, k, Hkv, d), r(S, k, Hkv, d)


def test_one_token_verify_is_the_decode_step(C):
    prefix, gen = [300, 17, 129], [5, 0, 40]
    a, _ = _filled(C, prefix, gen, 16, 4, 128, 40, 81)
    b, _ = _filled(C, prefix, gen, 16, 4, 128, 40, 81)
    q, kn, vn = _drafts(3, 1, 16, 4, 128, 82)
    say("verify k=1 vs decode")
    oa = torch.empty(3, 1, 16, 128, dtype=torch.bfloat16, device="cuda")
    ob = torch.empty(3, 16, 128, dtype=torch.bfloat16, device="cuda")
    a.verify(q.cuda(), kn.cuda(), vn.cuda(), oa, C.workspace(a.verify_workspace_size(1, 16), "cuda"))
    b.decode(q[:, 0].contiguous().cuda(), ob, C.workspace(b.decode_workspace_size(16), "cuda"),
             k_new=kn[:, 0].contiguous().cuda(), v_new=vn[:, 0].contiguous().cuda())
    torch.cuda.synchronize()
    assert torch.equal(oa[:, 0], ob)
    assert [a.seq_len(s) for s in range(3)] == [b.seq_len(s) for s in range(3)]
    a.close()
    b.close()


# rows per kv head = g * k: up to 4 take the per-row VALU kernel, more the
# MFMA kernel (32 rows per workgroup: 72 rows are three chunks, the last
# ragged; 64 drafts is the largest verify step)
# At 40 pages per sequence (5 splits) the splits are merged on chip; the
# cases at 80 (10 splits) take the merge kernel.
CASES = [(g, k, d, 40) for g, k in ((1, 3), (2, 2), (1, 8), (2, 3), (4, 2), (4, 4), (8, 4),
                                    (4, 16), (8, 9), (1, 64)) for d in (128,)]
CASES += [(4, 4, 64, 40), (2, 2, 64, 40)]
CASES += [(4, 4, 128, 80), (8, 9, 128, 80), (1, 64, 128, 80), (2, 3, 64, 80)]


@pytest.mark.parametrize("g,k,d,mp", CASES, ids=[f"g{g}-k{k}-d{d}-mp{mp}" for g, k, d, mp in CASES])
def test_verify_against_oracle(C, g, k, d, mp):
    Hkv = 2
    Hq = g * Hkv
    prefix, gen = [1, 90, 400, 33], [0, 7, 100, 16]
    cache, oc = _filled(C, prefix, gen, Hq, Hkv, d, mp, 100 + g + k)
    assert (cache.decode_schedule(Hq, k).waves_per_group > 0) == (mp == 40)
    q, kn, vn = _drafts(4, k, Hq, Hkv, d, 200 + g + k)
    out = torch.empty(4, k, Hq, d, dtype=torch.bfloat16, device="cuda")
    ws = C.workspace(cache.verify_workspace_size(k, Hq), "cuda")
    say("verify", g, k, d)
    cache.verify(q.cuda(), kn.cuda(), vn.cuda(), out, ws)
    torch.cuda.synchronize()
    ref = V.verify_step(oc, f64(q), f64(kn), f64(vn))
    assert rel(f64(out), ref) <= TOL
    assert [cache.seq_len(s) for s in range(4)] == [a + b + k for a, b in zip(prefix, gen)]
    assert f64(cache.seq_lens).astype(int).tolist() == [cache.seq_len(s) for s in range(4)]
    # rewind: keep the first accepted drafts of each stream, then decode one
    # more token behind the kept rows
    keep = [0, 1, k, k // 2]
    for s in range(4):
        new_len = prefix[s] + gen[s] + keep[s]
        cache.truncate(s, new_len)
        oc.k[s], oc.v[s] = oc.k[s][:new_len], oc.v[s][:new_len]
    q2, kn2, vn2 = _drafts(4, 1, Hq, Hkv, d, 300 + g + k)
    out2 = torch.empty(4, Hq, d, dtype=torch.bfloat16, device="cuda")
    cache.decode(q2[:, 0].contiguous().cuda(), out2,
                 C.workspace(cache.decode_workspace_size(Hq), "cuda"),
                 k_new=kn2[:, 0].contiguous().cuda(), v_new=vn2[:, 0].contiguous().cuda())
    torch.cuda.synchronize()
    assert rel(f64(out2), O.decode_step(oc, f64(q2[:, 0]), f64(kn2[:, 0]), f64(vn2[:, 0]))) <= TOL
    cache.close()


def test_verify_serving_decode_workload(C):
    """The serving-decode workload (64 sequences of p = 4096 plus up to 1024
    generated rows, Hq 32 / Hkv 8) verifying 4 drafts per sequence."""
    sh = W.DECODE
    di = W.decode_inputs(sh)
    S, Hq, Hkv, d = sh.n_seqs, sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    mp = di.max_pages_per_seq + 1                     # room for the drafts
    perm = torch.randperm(S * mp, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    cache = C.PagedCache(S, Hkv, d, mp, S * mp, perm.view(S, mp), "cuda")
    oc = O.DenseCache(S, Hkv, d)
    kc, vc = di.k_cart.cuda(), di.v_cart.cuda()
    kcf, vcf = f64(di.k_cart), f64(di.v_cart)
    say("verify, serving-decode workload: writing")
    for s in range(S):
        cache.write(s, kc, vc)
        oc.write(s, kcf, vcf)
        if di.generated[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    q, kn, vn = _drafts(S, 4, Hq, Hkv, d, 6)
    out = torch.empty(S, 4, Hq, d, dtype=torch.bfloat16, device="cuda")
    say("verify, serving-decode workload: step")
    cache.verify(q.cuda(), kn.cuda(), vn.cuda(), out,
                 C.workspace(cache.verify_workspace_size(4, Hq), "cuda"))
    torch.cuda.synchronize()
    assert rel(f64(out), V.verify_step(oc, f64(q), f64(kn), f64(vn))) <= TOL
    cache.close()


@pytest.mark.parametrize("g", [4, 8])
def test_decode_skips_pages_outside_the_pool(C, g):
    """Block-table entries outside [0, n_pages) are skipped: the decode
    attends over the rows of the valid pages only (they read as zeros and
    are masked, never dereferenced)."""
    Hkv, d = 2, 128
    Hq = g * Hkv
    prefix, gen = [300, 129], [20, 0]
    cache, _ = _filled(C, prefix, gen, Hq, Hkv, d, 40, 500 + g)
    di = W.decode_inputs_ragged(prefix, gen, Hq, Hkv, d, 40, seed=500 + g)
    # sequence 0 loses logical page 3 (an id past the pool) and page 7 (a
    # negative id); its other 18 pages stay
    cache.block_table[0, 3] = di.n_pages + 5
    cache.block_table[0, 7] = -1
    keep = np.ones(prefix[0] + gen[0], dtype=bool)
    keep[48:64] = False
    keep[112:128] = False
    oc = O.DenseCache(2, Hkv, d)
    k0 = np.concatenate([f64(di.k_cart[0]), f64(di.k_gen[0])])
    v0 = np.concatenate([f64(di.v_cart[0]), f64(di.v_gen[0])])
    oc.write(0, k0[keep], v0[keep])
    oc.write(1, f64(di.k_cart[1]), f64(di.v_cart[1]))
    out = torch.empty(2, Hq, d, dtype=torch.bfloat16, device="cuda")
    say("decode with pages outside the pool", g)
    cache.decode(di.q.cuda(), out, C.workspace(cache.decode_workspace_size(Hq), "cuda"))
    torch.cuda.synchronize()
    ref = O.decode_step(oc, f64(di.q))
    assert rel(f64(out), ref) <= TOL
