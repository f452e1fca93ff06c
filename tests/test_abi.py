"""Host-side tests of the libcartattn C ABI (no GPU needed).

Every argument check runs on the host before any HIP call, so each call here
is built to FAIL validation: no test passes a made-up pointer to a call that
would launch a kernel.
"""

import ctypes
import pathlib
import re

import pytest

from long_context_kv_amd import cartattn as C

ROOT = pathlib.Path(__file__).resolve().parents[1]
L = C.lib()
FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)
MIS = 0x10004           # misaligned


def _declared_functions():
    src = (ROOT / "include" / "cartattn.h").read_text()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(cart_\w+)\s*\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(C.EXPORTS) == names


def _shape(**kw):
    base = dict(batch=1, q_seq=16, p=8, frozen_rows=1, n_q_heads=4, n_kv_heads=2,
                head_dim=64, scale=0.0, tok_dtype=C.CART_BF16, row_dtype=C.CART_F32)
    base.update(kw)
    return C.AttnShape(**base)


def _fwd(shape, q=FAKE, kt=FAKE, vt=FAKE, kc=FAKE, vc=FAKE, out=FAKE, lse=FAKE, ws=FAKE,
         ws_bytes=1 << 30):
    return L.cart_attn_fwd(ctypes.byref(shape), q, kt, vt, kc, vc, out, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), C.CART_ERR_INVALID_ARG),
    (dict(q_seq=0), C.CART_ERR_INVALID_ARG),
    (dict(p=-1), C.CART_ERR_INVALID_ARG),
    (dict(frozen_rows=9), C.CART_ERR_INVALID_ARG),
    (dict(frozen_rows=-1), C.CART_ERR_INVALID_ARG),
    (dict(n_q_heads=5), C.CART_ERR_INVALID_ARG),
    (dict(n_kv_heads=0), C.CART_ERR_INVALID_ARG),
    (dict(head_dim=96), C.CART_ERR_UNSUPPORTED),
    (dict(head_dim=256), C.CART_ERR_UNSUPPORTED),
    (dict(scale=-1.0), C.CART_ERR_INVALID_ARG),
    (dict(scale=float("inf")), C.CART_ERR_INVALID_ARG),
    (dict(scale=float("nan")), C.CART_ERR_INVALID_ARG),
    (dict(tok_dtype=7), C.CART_ERR_INVALID_ARG),
    (dict(tok_dtype=C.CART_F32, row_dtype=C.CART_BF16), C.CART_ERR_UNSUPPORTED),
    (dict(batch=4096, q_seq=1 << 20, n_q_heads=64, n_kv_heads=8), C.CART_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    assert _fwd(_shape(**kw)) == status
    assert L.cart_attn_workspace_size(ctypes.byref(_shape(**kw)), 0) == 0
    assert L.cart_last_error()


def test_fwd_pointer_checks():
    s = _shape()
    assert _fwd(s, q=None) == C.CART_ERR_INVALID_ARG
    assert _fwd(s, q=MIS) == C.CART_ERR_ALIGNMENT
    assert _fwd(s, kc=None) == C.CART_ERR_INVALID_ARG     # p > 0 needs the cartridge
    assert _fwd(s, lse=None) == C.CART_ERR_INVALID_ARG
    assert _fwd(s, out=MIS) == C.CART_ERR_ALIGNMENT
    assert b"out" in L.cart_last_error()


def test_workspace_checks():
    # a shape small enough that the forward needs split partials
    s = _shape(batch=1, q_seq=64, p=4096, n_q_heads=2, n_kv_heads=1, head_dim=128)
    need = L.cart_attn_workspace_size(ctypes.byref(s), 0)
    assert need > 0
    assert _fwd(s, ws=None) == C.CART_ERR_WORKSPACE
    assert _fwd(s, ws_bytes=need - 1) == C.CART_ERR_WORKSPACE
    assert _fwd(s, ws=MIS, ws_bytes=need) == C.CART_ERR_ALIGNMENT
    need_b = L.cart_attn_workspace_size(ctypes.byref(s), 1)
    assert need_b >= 64 * 2 * 128 * 4      # at least the f32 dQ accumulator
    r = L.cart_attn_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, FAKE, FAKE, 0, FAKE, need_b - 256, None)
    assert r == C.CART_ERR_WORKSPACE


def test_bwd_pointer_checks():
    s = _shape()
    args = [FAKE] * 13
    for i in range(13):
        a = list(args)
        a[i] = None
        r = L.cart_attn_bwd(ctypes.byref(s), *a, 0, FAKE, 1 << 30, None)
        assert r == C.CART_ERR_INVALID_ARG, i
    # p = 0: cartridge pointers may be NULL, but frozen_rows must then be 0
    s0 = _shape(p=0, frozen_rows=1)
    assert _fwd(s0, kc=None, vc=None) == C.CART_ERR_INVALID_ARG


def test_rope_validation():
    f = L.cart_rope_tokens
    assert f(FAKE, FAKE, 5, 1, 1, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(FAKE, FAKE, C.CART_BF16, 1, 1, 4, 2, 80, 0, None, 1e6, 0, None) == C.CART_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, C.CART_BF16, 1, 1, 4, 2, 64, 0, None, 0.0, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(FAKE, FAKE, C.CART_BF16, 1, 1, 4, 2, 64, -1, None, 1e6, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(FAKE, FAKE, C.CART_BF16, -1, 1, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(None, FAKE, C.CART_BF16, 1, 1, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(MIS, None, C.CART_BF16, 1, 1, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_ERR_ALIGNMENT
    assert f(FAKE, MIS, C.CART_BF16, 1, 1, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_ERR_ALIGNMENT
    assert f(FAKE, FAKE, C.CART_BF16, 1, 1, 4, 0, 64, 0, None, 1e6, 0, None) == C.CART_ERR_INVALID_ARG
    assert f(FAKE, None, C.CART_BF16, 1, 1, 4, 2, 64, 0, FAKE + 2, 1e6, 0, None) == C.CART_ERR_ALIGNMENT
    # empty input is a successful no-op (nothing is launched)
    assert f(None, None, C.CART_BF16, 0, 5, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_OK
    assert f(None, None, C.CART_BF16, 3, 0, 4, 2, 64, 0, None, 1e6, 0, None) == C.CART_OK


def _desc(**kw):
    base = dict(n_seqs=2, n_kv_heads=2, head_dim=64, page_size=16, max_pages_per_seq=4,
                n_pages=8, dtype=C.CART_BF16, k_pages=FAKE, v_pages=FAKE, block_table=FAKE,
                seq_lens=FAKE)
    base.update(kw)
    return C.CacheDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_seqs=0), C.CART_ERR_INVALID_ARG),
    (dict(n_pages=0), C.CART_ERR_INVALID_ARG),
    (dict(head_dim=100), C.CART_ERR_UNSUPPORTED),
    (dict(page_size=32), C.CART_ERR_UNSUPPORTED),
    (dict(dtype=C.CART_F32), C.CART_ERR_UNSUPPORTED),
    (dict(k_pages=None), C.CART_ERR_INVALID_ARG),
    (dict(v_pages=MIS), C.CART_ERR_ALIGNMENT),
    (dict(block_table=None), C.CART_ERR_INVALID_ARG),
    (dict(seq_lens=None), C.CART_ERR_INVALID_ARG),
])
def test_cache_create_validation(kw, status):
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(_desc(**kw)), ctypes.byref(h)) == status
    assert not h.value


def test_cache_host_rules():
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(_desc()), ctypes.byref(h)) == C.CART_OK
    try:
        assert L.cart_cache_seq_len(h, 0) == 0
        assert L.cart_cache_seq_len(h, 2) == -1
        # geometry locked to the cache
        r = L.cart_write_cache(h, 0, FAKE, FAKE, C.CART_F32, 8, 4, 64, None)
        assert r == C.CART_ERR_GEOMETRY
        r = L.cart_write_cache(h, 0, FAKE, FAKE, C.CART_F32, 8, 2, 128, None)
        assert r == C.CART_ERR_GEOMETRY
        # capacity is 4 pages x 16 rows
        r = L.cart_write_cache(h, 0, FAKE, FAKE, C.CART_F32, 65, 2, 64, None)
        assert r == C.CART_ERR_CACHE_FULL
        assert L.cart_append_cache(h, 1, FAKE, FAKE, C.CART_BF16, 100, 2, 64, None) == \
            C.CART_ERR_CACHE_FULL
        assert L.cart_write_cache(h, 5, FAKE, FAKE, C.CART_F32, 8, 2, 64, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_write_cache(h, 0, None, FAKE, C.CART_F32, 8, 2, 64, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_append_cache(h, 0, FAKE, FAKE, 9, 8, 2, 64, None) == C.CART_ERR_INVALID_ARG
        # nothing stored yet: an attend-only decode has no rows to attend over
        # (a geometry whose splits are merged on chip needs no workspace)
        ws = L.cart_decode_workspace_size(h, 4)
        assert ws == 0
        assert L.cart_decode(h, FAKE, None, None, 4, 0.0, FAKE, FAKE, ws, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_decode(h, FAKE, FAKE, None, 4, 0.0, FAKE, FAKE, ws, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_decode(h, FAKE, None, None, 3, 0.0, FAKE, FAKE, ws, None) == \
            C.CART_ERR_GEOMETRY
        assert L.cart_decode(h, FAKE, None, None, 32, 0.0, FAKE, FAKE, ws, None) == \
            C.CART_ERR_UNSUPPORTED
        assert L.cart_decode(h, None, FAKE, FAKE, 4, 0.0, FAKE, FAKE, ws, None) == \
            C.CART_ERR_INVALID_ARG
        assert L.cart_decode_workspace_size(h, 3) == 0
        assert L.cart_decode_workspace_size(None, 4) == 0
    finally:
        L.cart_cache_destroy(h)


def test_status_strings():
    for s in range(9):
        assert L.cart_status_string(s)
    assert L.cart_status_string(99) == b"unknown status"


@pytest.mark.timeout(30)
def test_workspace_sizes_of_the_workloads():
    """Planning is host code: every workload shape (and a few extremes) gets a
    workspace size promptly (no planning loop runs away), below 1 TiB."""
    from long_context_kv_amd import workloads as W
    shapes = [(s.batch, s.q_seq, s.p, s.n_q_heads, s.n_kv_heads, s.head_dim)
              for s in W.SHAPES.values() if hasattr(s, "q_seq")]
    shapes += [(1, 1, 0, 2, 2, 64), (64, 4096, 65536, 64, 8, 128), (1, 131072, 1, 8, 8, 128),
               (512, 32, 4, 32, 1, 128)]
    for (b, n, p, hq, hkv, d) in shapes:
        for tok, row in ((C.CART_BF16, C.CART_F32), (C.CART_BF16, C.CART_BF16),
                         (C.CART_F32, C.CART_F32)):
            s = _shape(batch=b, q_seq=n, p=p, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                       frozen_rows=min(1, p), tok_dtype=tok, row_dtype=row)
            fw = L.cart_attn_workspace_size(ctypes.byref(s), 0)
            bw = L.cart_attn_workspace_size(ctypes.byref(s), 1)
            assert 0 <= fw < (1 << 40) and 0 <= bw < (1 << 40), (b, n, p, hq, hkv, d, tok, row)


# Shapes of the GPU parity cases (name, B, n, p, Hq, Hkv, d) whose dK/dV
# schedule must cut key tiles into pieces, so the in-kernel reduction of a
# cut tile stays covered by the GPU tests; and shapes that must not.
CUT_SHAPES = [
    ("pieces-g4", 2, 200, 600, 8, 2, 128),
    ("pieces-d64", 2, 150, 500, 8, 2, 64),
    ("token-heavy", 1, 500, 16, 4, 2, 128),
    ("ragged-g4", 2, 77, 200, 8, 2, 128),
    ("g8", 1, 70, 130, 16, 2, 128),
]
UNCUT_SHAPES = [
    ("units-1", 1, 20, 100, 1, 1, 128),
    ("units-2", 1, 40, 130, 2, 1, 128),
    ("units-3-ragged", 1, 70, 260, 3, 1, 128),
]


def _sched(B, n, p, Hq, Hkv, d, tok=C.CART_BF16, row=C.CART_F32):
    return C.cart_attn_schedule_query(_shape(batch=B, q_seq=n, p=p, n_q_heads=Hq,
                                             n_kv_heads=Hkv, head_dim=d, frozen_rows=min(1, p),
                                             tok_dtype=tok, row_dtype=row))


@pytest.mark.parametrize("case", CUT_SHAPES, ids=[c[0] for c in CUT_SHAPES])
def test_schedule_cuts_key_tiles(case):
    s = _sched(*case[1:])
    assert s.bwd_cart_pieces > 1 and s.bwd_tok_pieces_max > 1, case[0]
    # the grid holds every piece: cartridge tiles x pieces + the token pieces
    assert s.bwd_kv_grid >= case[5] * (s.bwd_cart_tiles * s.bwd_cart_pieces +
                                       case[1] * s.bwd_tok_tiles)


@pytest.mark.parametrize("case", UNCUT_SHAPES, ids=[c[0] for c in UNCUT_SHAPES])
def test_schedule_uncut_small_pipelines(case):
    s = _sched(*case[1:])
    assert s.bwd_cart_pieces == 1 and s.bwd_tok_pieces_max == 1, case[0]


def test_schedule_of_the_workloads():
    from long_context_kv_amd import workloads as W
    c2 = _sched(1, 1024, 2048, 16, 8, 128)
    # the small layer splits the key range of the forward and of the dQ kernel
    assert c2.fwd_key_splits > 1 and c2.bwd_dq_key_splits > 1
    assert c2.fwd_grid >= 512
    for sh in (W.QWEN3_8B, W.LONG):
        s = _sched(sh.batch, sh.q_seq, sh.p, sh.n_q_heads, sh.n_kv_heads, sh.head_dim)
        assert s.fwd_key_splits == 1 and s.bwd_dq_key_splits == 1, sh.name
        assert s.bwd_cart_tiles == (sh.p + 127) // 128
        assert s.bwd_tok_tiles == (sh.q_seq + 127) // 128
    f32 = _sched(1, 16, 8, 4, 2, 64, C.CART_F32, C.CART_F32)
    assert f32.bwd_dq_grid == 0 and f32.bwd_kv_grid >= 2


def test_schedule_validation():
    bad = ctypes.byref(_shape(batch=0))
    out = C.AttnSchedule()
    assert L.cart_attn_schedule_query(bad, ctypes.byref(out)) == C.CART_ERR_INVALID_ARG
    assert L.cart_attn_schedule_query(ctypes.byref(_shape()), None) == C.CART_ERR_INVALID_ARG


def test_qk_norm_rope_validation():
    f, b = L.cart_qk_norm_rope, L.cart_qk_norm_rope_bwd
    ok = dict(dt=C.CART_BF16, B=1, S=4, Hq=4, Hkv=2, d=64, eps=1e-6, base=0, offs=None, th=1e6)

    def fw(q=FAKE, k=FAKE, qo=FAKE, ko=FAKE, wq=FAKE, wk=FAKE, **kw):
        a = dict(ok, **kw)
        return f(q, k, qo, ko, wq, wk, a["dt"], a["B"], a["S"], a["Hq"], a["Hkv"], a["d"],
                 a["eps"], a["base"], a["offs"], a["th"], None)

    assert fw(dt=3) == C.CART_ERR_INVALID_ARG
    assert fw(d=96) == C.CART_ERR_UNSUPPORTED
    assert fw(eps=0.0) == C.CART_ERR_INVALID_ARG
    assert fw(th=-1.0) == C.CART_ERR_INVALID_ARG
    assert fw(base=-3) == C.CART_ERR_INVALID_ARG
    assert fw(wk=None) == C.CART_ERR_INVALID_ARG          # keys given without their weights
    assert fw(q=None) == C.CART_ERR_INVALID_ARG
    assert fw(wq=MIS) == C.CART_ERR_ALIGNMENT
    assert fw(ko=None) == C.CART_ERR_INVALID_ARG
    assert fw(offs=FAKE + 2) == C.CART_ERR_ALIGNMENT
    assert fw(q=None, S=0) == C.CART_OK                   # empty: nothing launched
    # backward: the input gradient may not overwrite the inputs
    r = b(FAKE, None, FAKE + 16, None, FAKE, None, FAKE, None, C.CART_BF16, 1, 4, 4, 2, 64,
          1e-6, 0, None, 1e6, None)
    assert r == C.CART_ERR_INVALID_ARG and b"overwrite" in L.cart_last_error()
    r = b(FAKE, None, None, None, FAKE + 16, None, FAKE, None, C.CART_BF16, 1, 4, 4, 2, 64,
          1e-6, 0, None, 1e6, None)
    assert r == C.CART_ERR_INVALID_ARG


def test_adam_rows_validation():
    f = L.cart_adam_rows

    def call(rows=FAKE, grad=FAKE, m=FAKE, v=FAKE, xb=None, n=8, e=64, fr=1, t=1, lr=2e-2,
             b1=0.9, b2=0.999, eps=1e-8):
        return f(rows, grad, m, v, xb, n, e, fr, t, lr, b1, b2, eps, None)

    assert call(e=6) == C.CART_ERR_UNSUPPORTED
    assert call(n=-1) == C.CART_ERR_INVALID_ARG
    assert call(fr=9) == C.CART_ERR_INVALID_ARG
    assert call(t=0) == C.CART_ERR_INVALID_ARG
    assert call(lr=-1.0) == C.CART_ERR_INVALID_ARG
    assert call(b1=1.0) == C.CART_ERR_INVALID_ARG
    assert call(b2=-0.1) == C.CART_ERR_INVALID_ARG
    assert call(eps=0.0) == C.CART_ERR_INVALID_ARG
    assert call(m=None) == C.CART_ERR_INVALID_ARG
    assert call(xb=MIS) == C.CART_ERR_ALIGNMENT
    assert call(rows=None, n=0, fr=0) == C.CART_OK         # empty: nothing launched


def test_rows_to_bf16_validation():
    f = L.cart_rows_to_bf16

    def call(k=FAKE, v=FAKE + 4096, kb=FAKE + 8192, vb=FAKE + 12288, n=8, e=64):
        return f(k, v, kb, vb, n, e, None)

    assert call(e=6) == C.CART_ERR_UNSUPPORTED
    assert call(n=-1) == C.CART_ERR_INVALID_ARG
    assert call(e=0) == C.CART_ERR_INVALID_ARG
    assert call(k=None) == C.CART_ERR_INVALID_ARG
    assert call(vb=None) == C.CART_ERR_INVALID_ARG
    assert call(kb=MIS) == C.CART_ERR_ALIGNMENT
    assert call(kb=FAKE + 1024) == C.CART_ERR_INVALID_ARG      # k_bf16 inside k
    assert call(vb=FAKE + 8192 + 512) == C.CART_ERR_INVALID_ARG  # outputs overlap
    assert b"overlap" in L.cart_last_error()
    assert call(k=None, v=None, kb=None, vb=None, n=0) == C.CART_OK   # empty: nothing launched


def _parts(rows, frozen, ptr=FAKE):
    n = len(rows)
    kp = (ctypes.c_void_p * n)(*[ptr if r else None for r in rows])
    vp = (ctypes.c_void_p * n)(*[ptr if r else None for r in rows])
    p = C.Parts(n, (ctypes.c_int32 * n)(*rows), (ctypes.c_int32 * n)(*frozen), kp, vp)
    p._keep = (kp, vp)
    return p


def test_parts_validation():
    assert L.cart_parts_rows(ctypes.byref(_parts([3, 0, 5], [1, 0, 2]))) == 8
    assert L.cart_parts_rows(ctypes.byref(_parts([3, -1], [1, 0]))) == -1
    assert L.cart_parts_rows(ctypes.byref(_parts([3, 2], [1, 3]))) == -1
    assert L.cart_parts_rows(ctypes.byref(_parts([1] * 65, [0] * 65))) == -1
    assert L.cart_parts_rows(None) == -1
    comp = L.cart_compose_rows
    assert comp(ctypes.byref(_parts([3, 5], [1, 1])), C.CART_BF16, 2, 64, FAKE, FAKE,
                C.CART_F32, None) == C.CART_ERR_UNSUPPORTED
    assert comp(ctypes.byref(_parts([3, 5], [1, 1], ptr=MIS)), C.CART_F32, 2, 64, FAKE, FAKE,
                C.CART_BF16, None) == C.CART_ERR_ALIGNMENT
    assert comp(ctypes.byref(_parts([3, 5], [1, 1])), C.CART_F32, 2, 80, FAKE, FAKE,
                C.CART_BF16, None) == C.CART_ERR_UNSUPPORTED
    assert comp(ctypes.byref(_parts([3, 5], [1, 1])), C.CART_F32, 2, 64, None, FAKE,
                C.CART_BF16, None) == C.CART_ERR_INVALID_ARG
    assert comp(ctypes.byref(_parts([0, 0], [0, 0], ptr=None)), C.CART_F32, 2, 64, None, None,
                C.CART_BF16, None) == C.CART_OK          # nothing to compose
    # the composed backward wants the shape's p to be the composed length
    s = _shape(p=9)
    r = L.cart_attn_bwd_composed(ctypes.byref(s), ctypes.byref(_parts([3, 5], [1, 1])),
                                 *([FAKE] * 13), 0, FAKE, 1 << 30, None)
    assert r == C.CART_ERR_INVALID_ARG and b"parts" in L.cart_last_error()


def test_write_composed_cache_refusals():
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(_desc()), ctypes.byref(h)) == C.CART_OK
    try:
        w = L.cart_write_composed_cache
        # 4 pages x 16 rows = 64 rows: 40 + 30 do not fit; nothing is appended
        assert w(h, 0, ctypes.byref(_parts([40, 30], [1, 1])), C.CART_F32, 2, 64, None) == \
            C.CART_ERR_CACHE_FULL
        assert L.cart_cache_seq_len(h, 0) == 0
        assert w(h, 0, ctypes.byref(_parts([4, 3], [1, 1])), C.CART_F32, 4, 64, None) == \
            C.CART_ERR_GEOMETRY
        assert w(h, 0, ctypes.byref(_parts([4, 3], [1, 1], ptr=None)), C.CART_F32, 2, 64,
                 None) == C.CART_ERR_INVALID_ARG
        assert w(h, 9, ctypes.byref(_parts([4, 3], [1, 1])), C.CART_F32, 2, 64, None) == \
            C.CART_ERR_INVALID_ARG
    finally:
        L.cart_cache_destroy(h)


def _decode_schedule(h, n_tokens, n_q_heads):
    out = C.DecodeSchedule()
    assert L.cart_decode_schedule_query(h, n_tokens, n_q_heads, ctypes.byref(out)) == C.CART_OK
    return out


@pytest.mark.parametrize("n_seqs,hkv,max_pages,hq", [
    (2, 2, 4, 4), (5, 2, 40, 8), (3, 2, 24, 4), (64, 8, 320, 32), (1, 8, 100, 64),
    (6, 8, 81, 32), (5, 2, 80, 16), (64, 8, 16384, 64), (1, 1, 1, 8)])
def test_decode_schedule_query(n_seqs, hkv, max_pages, hq):
    """The decode plan: a sequence's splits are merged on chip (one
    workgroup of a power-of-two count of waves, no workspace) when there are
    at most 8 of them, else by a merge kernel through the workspace; the
    workspace sizes the entry points report are the plan's."""
    d = _desc(n_seqs=n_seqs, n_kv_heads=hkv, head_dim=128, max_pages_per_seq=max_pages,
              n_pages=n_seqs * max_pages)
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(d), ctypes.byref(h)) == C.CART_OK
    try:
        for k in (1, 4, 64):
            sc = _decode_schedule(h, k, hq)
            pps, ms = sc.pages_per_split, sc.max_splits
            assert pps % 4 == 0 and 8 <= pps <= 256
            assert ms == -(-max_pages // pps) and (ms - 1) * pps < max_pages
            chunks = -(-(hq // hkv) * k // 32)
            if ms <= 8:
                w = sc.waves_per_group
                assert w in (1, 2, 4, 8) and w >= ms and (w == 1 or w < 2 * ms)
                assert sc.grid == n_seqs * hkv * chunks and sc.workspace_bytes == 0
            else:
                assert sc.waves_per_group == 0
                assert sc.grid == n_seqs * hkv * chunks * ms
                assert sc.workspace_bytes == n_seqs * k * hq * ms * (4 + 128) * 4
            want = (L.cart_decode_workspace_size(h, hq) if k == 1 else
                    L.cart_decode_verify_workspace_size(h, k, hq))
            assert sc.workspace_bytes == want
        bad = C.DecodeSchedule()
        assert L.cart_decode_schedule_query(None, 1, hq, ctypes.byref(bad)) == C.CART_ERR_INVALID_ARG
        assert L.cart_decode_schedule_query(h, 1, hq, None) == C.CART_ERR_INVALID_ARG
        assert L.cart_decode_schedule_query(h, 0, hq, ctypes.byref(bad)) == C.CART_ERR_INVALID_ARG
        assert L.cart_decode_schedule_query(h, 65, hq, ctypes.byref(bad)) == C.CART_ERR_INVALID_ARG
        assert L.cart_decode_schedule_query(h, 1, hkv + 1 if hkv > 1 else 0,
                                            ctypes.byref(bad)) == C.CART_ERR_INVALID_ARG
    finally:
        L.cart_cache_destroy(h)


def test_verify_and_truncate_host_rules():
    h = ctypes.c_void_p()
    assert L.cart_cache_create(ctypes.byref(_desc()), ctypes.byref(h)) == C.CART_OK
    try:
        ws = L.cart_decode_verify_workspace_size(h, 4, 4)
        assert ws == 0 == L.cart_decode_workspace_size(h, 4)   # merged on chip
        assert L.cart_decode_verify_workspace_size(h, 0, 4) == 0
        assert L.cart_decode_verify_workspace_size(h, 65, 4) == 0
        # with more than 8 splits per sequence the partials go through the
        # workspace: 4 tokens, 4x the partials of one
        h2 = ctypes.c_void_p()
        assert L.cart_cache_create(ctypes.byref(_desc(max_pages_per_seq=100, n_pages=200)),
                                   ctypes.byref(h2)) == C.CART_OK
        try:
            ws2 = L.cart_decode_verify_workspace_size(h2, 4, 4)
            assert ws2 == 4 * L.cart_decode_workspace_size(h2, 4) > 0
            assert L.cart_decode_verify(h2, FAKE, FAKE, FAKE, 4, 4, 0.0, FAKE, FAKE, ws2 - 1,
                                        None) == C.CART_ERR_WORKSPACE
            assert L.cart_decode_verify(h2, FAKE, FAKE, FAKE, 4, 4, 0.0, FAKE, None, ws2,
                                        None) == C.CART_ERR_WORKSPACE
        finally:
            L.cart_cache_destroy(h2)
        v = L.cart_decode_verify
        # drafts are appended: k_new / v_new are required
        assert v(h, FAKE, None, None, 4, 4, 0.0, FAKE, FAKE, ws, None) == C.CART_ERR_INVALID_ARG
        assert v(h, FAKE, FAKE, FAKE, 0, 4, 0.0, FAKE, FAKE, ws, None) == C.CART_ERR_INVALID_ARG
        assert v(h, FAKE, FAKE, FAKE, 4, 3, 0.0, FAKE, FAKE, ws, None) == C.CART_ERR_GEOMETRY
        # capacity is 64 rows: 65 drafts at once do not fit (refused as too many)
        assert v(h, FAKE, FAKE, FAKE, 65, 4, 0.0, FAKE, FAKE, 1 << 30, None) == \
            C.CART_ERR_INVALID_ARG
        # truncation only shortens
        assert L.cart_cache_truncate(h, 0, 1, None) == C.CART_ERR_INVALID_ARG
        assert L.cart_cache_truncate(h, 0, -1, None) == C.CART_ERR_INVALID_ARG
        assert L.cart_cache_truncate(h, 7, 0, None) == C.CART_ERR_INVALID_ARG
    finally:
        L.cart_cache_destroy(h)


def test_long_cartridge_schedule_cuts_token_tiles_only():
    """On the long-cartridge layer the dK/dV plan deals every cartridge tile
    whole (256 units: four rounds of 256 CUs) and cuts the larger causal
    token tiles, which come last, into up to three pieces, so that the last
    round evens out; the tiles' pieces are reduced in the kernel."""
    s = _sched(1, 4096, 16384, 16, 8, 128)
    assert s.bwd_cart_pieces == 1 and s.bwd_units_per_piece == 256
    assert s.bwd_tok_pieces_max == 3
    assert s.bwd_kv_grid > (s.bwd_cart_tiles + s.bwd_tok_tiles) * 8


@pytest.mark.parametrize("B,n,p,Hq,Hkv,d", [
    (1, 4096, 16384, 16, 8, 128), (4, 2048, 4096, 32, 8, 128), (1, 1024, 2048, 16, 8, 128),
    (2, 200, 600, 8, 2, 128), (1, 500, 16, 4, 2, 128), (3, 77, 0, 6, 3, 64),
    (1, 8192, 1024, 8, 1, 128), (2, 3000, 500, 12, 4, 64), (1, 1, 9, 4, 2, 64)])
def test_dkdv_grid_follows_the_piece_rule(B, n, p, Hq, Hkv, d):
    """The dK/dV grid is the sum of the pieces the kernel derives for its
    block ids: every cartridge tile in the same number of pieces, token tile
    t (units g * (query tiles from 4 t on) per sequence) in
    ceil(units / token target) pieces, the token target at most the
    cartridge one."""
    s = _sched(B, n, p, Hq, Hkv, d)
    g, nqt, n_tt = Hq // Hkv, -(-n // 32), -(-n // 128)
    tt, tc = s.bwd_tok_units_per_piece, s.bwd_units_per_piece
    assert 1 <= tt and (p == 0 or tt <= tc)
    tok = [-(-(g * (nqt - 4 * t)) // tt) for t in range(n_tt)]
    n_ct = -(-p // 128)
    assert s.bwd_cart_tiles == n_ct and s.bwd_tok_tiles == n_tt
    if n_ct:
        assert s.bwd_cart_pieces == -(-(B * g * nqt) // tc)
    assert s.bwd_tok_pieces_max == max(tok + [1])
    assert s.bwd_kv_grid == Hkv * (n_ct * s.bwd_cart_pieces + B * sum(tok))


def test_window_schedule_and_validation():
    assert _fwd(_shape(window=-1)) == C.CART_ERR_INVALID_ARG
    full = _sched(1, 4096, 16384, 16, 8, 128)
    s = C.cart_attn_schedule_query(_shape(batch=1, q_seq=4096, p=16384, n_q_heads=16,
                                          n_kv_heads=8, head_dim=128, window=1024))
    # a 1024-row window leaves most of the cartridge unseen: one piece per
    # key tile, with far fewer (batch, head, query-tile) units
    tiles = (s.bwd_cart_tiles + s.bwd_tok_tiles) * 8
    assert s.bwd_kv_grid == tiles and s.bwd_cart_tiles == full.bwd_cart_tiles
    assert 3 * s.bwd_units_per_piece < full.bwd_units_per_piece
    assert full.bwd_kv_grid >= tiles
    wide = C.cart_attn_schedule_query(_shape(batch=1, q_seq=4096, p=16384, n_q_heads=16,
                                             n_kv_heads=8, head_dim=128, window=20480))
    assert wide.bwd_kv_grid == full.bwd_kv_grid     # a window reaching every row is none


def test_packed_validation_and_schedule():
    lens = (ctypes.c_int32 * 3)(10, 0, 5)
    s = _shape(batch=3, q_seq=10)
    s.seg_lens = lens
    assert _fwd(s) == C.CART_ERR_INVALID_ARG            # a segment of length 0
    lens[1] = 11
    assert _fwd(s) == C.CART_ERR_INVALID_ARG            # longer than q_seq
    lens[1] = 7
    assert L.cart_attn_workspace_size(ctypes.byref(s), 1) > 0
    many = (ctypes.c_int32 * 65)(*([1] * 65))
    s65 = _shape(batch=65, q_seq=1)
    s65.seg_lens = many
    assert _fwd(s65) == C.CART_ERR_UNSUPPORTED
    r = L.cart_rope_tokens_packed(FAKE, None, C.CART_BF16, 0, lens, 4, 2, 64, 0, 1e6, 0, None)
    assert r == C.CART_ERR_INVALID_ARG
    r = L.cart_rope_tokens_packed(FAKE, None, C.CART_BF16, 3, None, 4, 2, 64, 0, 1e6, 0, None)
    assert r == C.CART_ERR_INVALID_ARG
    # packed segments of equal length schedule exactly like the batch
    eq = (ctypes.c_int32 * 4)(*([512] * 4))
    sp = _shape(batch=4, q_seq=512, p=2048, n_q_heads=16, n_kv_heads=8, head_dim=128)
    sp.seg_lens = eq
    sb = _shape(batch=4, q_seq=512, p=2048, n_q_heads=16, n_kv_heads=8, head_dim=128)
    a, b = C.cart_attn_schedule_query(sp), C.cart_attn_schedule_query(sb)
    assert [getattr(a, f) for f, _ in a._fields_] == [getattr(b, f) for f, _ in b._fields_]
    # ragged segments: fewer token tiles than the padded batch would have
    rag = (ctypes.c_int32 * 4)(512, 100, 30, 250)
    sr = _shape(batch=4, q_seq=512, p=2048, n_q_heads=16, n_kv_heads=8, head_dim=128)
    sr.seg_lens = rag
    assert C.cart_attn_schedule_query(sr).bwd_kv_grid < b.bwd_kv_grid
