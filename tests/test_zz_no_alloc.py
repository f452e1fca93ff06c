"""The allocation-free decode entry point, cart_decode_noalloc, against
cart_decode (the same step with a caller workspace) and the oracle.

The host-side checks run without a GPU; the GPU test calls both entry points
through the C ABI on two caches in a row, the second smaller than the first,
so the library's scratch is reused with a smaller geometry.
"""

import ctypes

import numpy as np
import pytest
import torch

from long_context_kv_amd import cartattn as C
from long_context_kv_amd import workloads as W
from oracle import cartattn_oracle as O
from tests._common import f64, rel, say

FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)
L = C.lib()


def test_noalloc_host_checks():
    assert L.cart_decode_noalloc_max_bytes() == 16 << 20
    # a geometry whose split partials exceed the scratch is refused before any
    # HIP call (the appended row gives every sequence one row to attend over);
    # 64 splits per sequence, so they are merged through the scratch
    desc = C.CacheDesc(64, 8, 128, 16, 16384, 64 * 16384, C.CART_BF16, FAKE, FAKE, FAKE, FAKE)
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(desc), ctypes.byref(h)) == C.CART_OK
    try:
        need = L.cart_decode_workspace_size(h, 64)
        assert need > L.cart_decode_noalloc_max_bytes()
        r = L.cart_decode_noalloc(h, FAKE, FAKE, FAKE, 64, 0.0, FAKE, None)
        assert r == C.CART_ERR_WORKSPACE
        assert b"scratch" in L.cart_last_error()
        # the other checks are cart_decode's
        assert L.cart_decode_noalloc(h, FAKE, None, None, 64, 0.0, FAKE, None) == \
            C.CART_ERR_INVALID_ARG                                   # no rows yet
        assert L.cart_decode_noalloc(h, FAKE, FAKE, FAKE, 60, 0.0, FAKE, None) == \
            C.CART_ERR_GEOMETRY
        assert L.cart_decode_noalloc(h, None, FAKE, FAKE, 64, 0.0, FAKE, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_decode_noalloc(None, FAKE, FAKE, FAKE, 64, 0.0, FAKE, None) == \
            C.CART_ERR_INVALID_ARG
    finally:
        L.cart_cache_destroy(h)


def _filled_cache(prefix, gen, Hq, Hkv, d, max_pages, seed):
    di = W.decode_inputs_ragged(prefix, gen, Hq, Hkv, d, max_pages, seed=seed)
    n = len(prefix)
    cache = C.PagedCache(n, Hkv, d, max_pages, di.n_pages, di.page_perm.view(n, max_pages),
                         "cuda")
    oc = O.DenseCache(n, Hkv, d)
    for s in range(n):
        cache.write(s, di.k_cart[s].cuda(), di.v_cart[s].cuda())
        oc.write(s, f64(di.k_cart[s]), f64(di.v_cart[s]))
        if gen[s]:
            cache.append(s, di.k_gen[s].cuda(), di.v_gen[s].cuda())
            oc.append(s, f64(di.k_gen[s]), f64(di.v_gen[s]))
    return cache, oc, di


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [
        # (prefix lengths, generated lengths, Hq, Hkv, d, max_pages, seed): the
        # second is smaller (fewer sequences, shorter, fewer heads)
        ([700, 33, 1200, 5, 64, 980], [50, 0, 80, 3, 200, 0], 32, 8, 128, 81, 71),
        ([40, 300, 9], [7, 0, 1], 8, 2, 64, 72, 72),
    ]
    for i, (prefix, gen, Hq, Hkv, d, mp, seed) in enumerate(cases):
        say("noalloc call", i, "seqs", len(prefix), "Hq", Hq, "d", d)
        cache, oc, di = _filled_cache(prefix, gen, Hq, Hkv, d, mp, seed)
        n = len(prefix)
        q = di.q.cuda()
        out_ws = torch.empty(n, Hq, d, dtype=torch.bfloat16, device="cuda")
        out_na = torch.full_like(out_ws, float("nan"))
        ws = C.workspace(cache.decode_workspace_size(Hq), "cuda")
        # more than 8 splits per sequence: the partials go through the scratch
        assert cache.decode_schedule(Hq).waves_per_group == 0
        assert 0 < cache.decode_workspace_size(Hq) <= C.decode_noalloc_max_bytes()
        cache.decode(q, out_ws, ws)
        cache.decode_noalloc(q, out_na)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), i
        assert rel(f64(out_na), O.decode_step(oc, f64(di.q))) <= 2e-2
        # an appending step through the allocation-free entry point
        lens = [cache.seq_len(s) for s in range(n)]
        cache.decode_noalloc(q, out_na, k_new=di.k_new.cuda(), v_new=di.v_new.cuda())
        torch.cuda.synchronize()
        assert [cache.seq_len(s) for s in range(n)] == [x + 1 for x in lens]
        ref = O.decode_step(oc, f64(di.q), f64(di.k_new), f64(di.v_new))
        assert rel(f64(out_na), ref) <= 2e-2
        cache.decode(q, out_ws, ws)           # same rows, workspace entry point
        cache.decode_noalloc(q, out_na)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), i
        cache.close()


@pytest.mark.gpu
def test_noalloc_with_splits_merged_on_chip():
    """A geometry of at most 8 splits per sequence needs no partials at all:
    the allocation-free call takes the same kernel, without the scratch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    prefix, gen, Hq, Hkv, d = [200, 1, 90], [9, 0, 30], 16, 4, 128
    say("noalloc on-chip merge")
    cache, oc, di = _filled_cache(prefix, gen, Hq, Hkv, d, 24, 73)
    assert cache.decode_schedule(Hq).waves_per_group > 0
    assert cache.decode_workspace_size(Hq) == 0
    out_ws = torch.empty(3, Hq, d, dtype=torch.bfloat16, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    q = di.q.cuda()
    cache.decode(q, out_ws, None)
    cache.decode_noalloc(q, out_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws)
    assert rel(f64(out_na), O.decode_step(oc, f64(di.q))) <= 2e-2
    cache.close()
