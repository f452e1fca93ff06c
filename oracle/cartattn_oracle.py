"""Plain CPU float64 oracle for cartridge attention.

TEST INFRASTRUCTURE ONLY. This module is the correctness reference that the
HIP library is checked against. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it. It shares no code with the GPU path and imports nothing from it.

Everything is the plain definition written out in numpy float64: dense masked
softmax attention per (batch, q-head), the softmax adjoint for the backward,
and a dense per-sequence KV store for serving. No blocking, no online
softmax, no fusion. Query rows are processed in chunks only to bound memory;
each chunk is the same plain computation.

Sources (titles of the pages the method is described on):

* "Cartridges: trained KV-prefix corpus compression" (Fucina guide), section
  "Semantics (pinned to the reference implementation)": per-layer cartridge
  K/V of shape [p, kv_head, d] in KV-cache space, keys already rotated at
  positions 0..p-1 and never rotated again; real tokens at RoPE positions
  p, p+1, ...; row 0 a frozen constant; attention over
  concat(sink, trainable, tokens) with the causal mask aligned to the end
  (source_offset = kv_seq - q_seq): all prefix rows are visible to each
  query, and among the tokens a query reaches itself and the earlier ones;
  the backward in f32 carries gradients through the concat into the
  trainable rows; for serving, an empty cache takes the p prefix rows in its
  own dtype, its length becomes p, and decoding resumes at position p.
* Same page, section "Evidence": gradcheck with kv_seq > q_seq and GQA;
  zero-training prefill equivalence; serving parity of decode behind the
  written prefix.
* "RIG minimal cognition engine implementation hand-off", section 5 (the
  cartridge file layout and its RoPE warning): a shifted base position
  silently corrupts attention.

Readings where the pages are silent:

* scale defaults to 1/sqrt(d);
* q-head h reads kv-head h // (Hq / Hkv) (contiguous GQA groups);
* RoPE pairs element k with k + d/2 ("rotate-half"), frequency
  theta**(-2k/d), angles in float64;
* the mask is inclusive: key row j is visible to query i iff j <= i + p;
* one cartridge per layer is shared by the whole batch, so its gradients are
  summed over batch and GQA group;
* rows below ``frozen_rows`` get an exact zero gradient;
* every float32 -> bfloat16 conversion rounds to nearest, ties to even;
* a decode step places the new token at position seq_len, appends its K/V
  first and then attends over every stored row (it sees itself).

Layouts: Q, O, dO, dQ are [B, n, Hq, d]; token K/V are [B, n, Hkv, d];
cartridge K/V are [p, Hkv, d]; LSE is [B, Hq, n] (natural log).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "default_scale",
    "rope_angles",
    "rope",
    "token_positions",
    "attn_fwd",
    "attn_bwd",
    "causal_prefill",
    "causal_prefill_bwd",
    "round_bf16",
    "DenseCache",
    "decode_step",
    "fd_grad",
]

# Query rows per chunk; bounds the dense score block to about
# _CHUNK * kv_seq float64 values per (batch, head).
_CHUNK = 1024


def default_scale(head_dim: int) -> float:
    """Softmax scale when the caller passes 0: 1/sqrt(d) (a reading; the
    pages do not state the scale)."""
    return 1.0 / np.sqrt(float(head_dim))


# --------------------------------------------------------------------------
# RoPE ("Semantics": real tokens sit at positions p, p+1, ...; cartridge
# keys are never rotated again).
# --------------------------------------------------------------------------

def rope_angles(positions, head_dim: int, theta: float):
    """cos and sin of pos * theta**(-2k/d) for k in [0, d/2), float64.

    positions: integer array of any shape. Returns two arrays of shape
    positions.shape + (d/2,).
    """
    half = head_dim // 2
    k = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * k / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    return np.cos(ang), np.sin(ang)


def rope(x, positions, theta: float, inverse: bool = False):
    """Rotate x[..., S, H, d] at per-row positions[..., S] (float64 result).

    Pair (k, k + d/2) is rotated by angle pos * theta_k; ``inverse`` rotates
    by -angle, which is the transpose (adjoint) of the forward rotation and
    is what carries a gradient back through RoPE.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    c, s = rope_angles(positions, d, theta)       # [..., S, half]
    c = c[..., None, :]                           # broadcast over heads
    s = s[..., None, :]
    if inverse:
        s = -s
    lo = x[..., :half]
    hi = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = lo * c - hi * s
    out[..., half:] = hi * c + lo * s
    return out


def token_positions(batch: int, seq: int, pos_base: int, pos_offsets=None):
    """Position of token (b, i) = pos_base + pos_offsets[b] + i."""
    pos = pos_base + np.arange(seq, dtype=np.int64)[None, :].repeat(batch, 0)
    if pos_offsets is not None:
        pos = pos + np.asarray(pos_offsets, dtype=np.int64)[:, None]
    return pos


# --------------------------------------------------------------------------
# Forward ("Semantics": concat(sink, trainable, tokens) along seq feeds the
# end-aligned causal grouped attention; "Evidence": kv_seq > q_seq, GQA).
# --------------------------------------------------------------------------

def _keys_for(b, kv, k_tok, v_tok, k_cart, v_cart):
    """Concatenated key/value rows [p + n, d] seen by kv-head kv of batch b."""
    K = np.concatenate([k_cart[:, kv, :], k_tok[b, :, kv, :]], axis=0)
    V = np.concatenate([v_cart[:, kv, :], v_tok[b, :, kv, :]], axis=0)
    return K, V


def _probs(Qc, K, rows, p, scale):
    """Softmax probabilities and LSE for query rows ``rows`` (plain, dense).

    Key row j is visible to query i iff j <= i + p, with p = kv_seq - q_seq.
    """
    S = scale * (Qc @ K.T)                        # [r, L]
    L = K.shape[0]
    j = np.arange(L)[None, :]
    visible = j <= (rows[:, None] + p)
    S = np.where(visible, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    lse = (m + np.log(l))[:, 0]
    return P, lse


def attn_fwd(q, k_tok, v_tok, k_cart, v_cart, scale: float = 0.0):
    """O and LSE of end-aligned causal GQA over concat(cartridge, tokens).

    All arrays are converted to float64 (exact for f32 and bf16 inputs).
    Returns (O [B, n, Hq, d], LSE [B, Hq, n]).
    """
    q = np.asarray(q, np.float64)
    k_tok = np.asarray(k_tok, np.float64)
    v_tok = np.asarray(v_tok, np.float64)
    k_cart = np.asarray(k_cart, np.float64)
    v_cart = np.asarray(v_cart, np.float64)
    B, n, Hq, d = q.shape
    p, Hkv = k_cart.shape[0], k_tok.shape[2]
    g = Hq // Hkv
    if scale == 0.0:
        scale = default_scale(d)
    O = np.zeros((B, n, Hq, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            K, V = _keys_for(b, kv, k_tok, v_tok, k_cart, v_cart)
            for r0 in range(0, n, _CHUNK):
                rows = np.arange(r0, min(n, r0 + _CHUNK))
                P, lse = _probs(q[b, rows, h, :], K, rows, p, scale)
                O[b, rows, h, :] = P @ V
                LSE[b, h, rows] = lse
    return O, LSE


# --------------------------------------------------------------------------
# Backward ("Semantics": the f32-KV backward routes gradients through the
# concat into the trainable rows; row 0 is frozen).
# --------------------------------------------------------------------------

def attn_bwd(q, k_tok, v_tok, k_cart, v_cart, dout, scale: float = 0.0,
             frozen_rows: int = 1):
    """Gradients of sum(O * dO) with respect to every input.

    Softmax adjoint per (b, h):  D = rowsum(dO * O);  dV = P^T dO;
    dP = dO V^T;  dS = P * (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
    Cartridge rows (j < p) are summed over batch and the group's q-heads;
    token rows are summed over the group's q-heads for their own batch.
    Rows below ``frozen_rows`` of the cartridge gradients are exactly zero.

    Returns (dq, dk_tok, dv_tok, dk_cart, dv_cart), float64, in the layouts
    of the corresponding inputs. No RoPE adjoint is applied here.
    """
    q = np.asarray(q, np.float64)
    k_tok = np.asarray(k_tok, np.float64)
    v_tok = np.asarray(v_tok, np.float64)
    k_cart = np.asarray(k_cart, np.float64)
    v_cart = np.asarray(v_cart, np.float64)
    dout = np.asarray(dout, np.float64)
    B, n, Hq, d = q.shape
    p, Hkv = k_cart.shape[0], k_tok.shape[2]
    g = Hq // Hkv
    if scale == 0.0:
        scale = default_scale(d)
    dq = np.zeros_like(q)
    dk_tok = np.zeros_like(k_tok)
    dv_tok = np.zeros_like(v_tok)
    dk_cart = np.zeros_like(k_cart)
    dv_cart = np.zeros_like(v_cart)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            K, V = _keys_for(b, kv, k_tok, v_tok, k_cart, v_cart)
            dK = np.zeros_like(K)
            dV = np.zeros_like(V)
            for r0 in range(0, n, _CHUNK):
                rows = np.arange(r0, min(n, r0 + _CHUNK))
                Qc = q[b, rows, h, :]
                dOc = dout[b, rows, h, :]
                P, _ = _probs(Qc, K, rows, p, scale)
                Oc = P @ V
                D = np.sum(dOc * Oc, axis=1, keepdims=True)
                dV += P.T @ dOc
                dP = dOc @ V.T
                dS = P * (dP - D)
                dq[b, rows, h, :] = scale * (dS @ K)
                dK += scale * (dS.T @ Qc)
            dk_cart[:, kv, :] += dK[:p]
            dv_cart[:, kv, :] += dV[:p]
            dk_tok[b, :, kv, :] += dK[p:]
            dv_tok[b, :, kv, :] += dV[p:]
    f = int(frozen_rows)
    dk_cart[:f] = 0.0
    dv_cart[:f] = 0.0
    return dq, dk_tok, dv_tok, dk_cart, dv_cart


# --------------------------------------------------------------------------
# Textbook causal attention (no cartridge): the reference the zero-training
# prefill-equivalence gate compares against ("Semantics", initialization;
# "Evidence", prefill equivalence).
# --------------------------------------------------------------------------

def causal_prefill(q, k, v, scale: float = 0.0):
    """Plain causal GQA over T tokens: query t sees keys 0..t.

    q [B, T, Hq, d], k/v [B, T, Hkv, d]. Returns (O, LSE).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hq, d = q.shape
    empty = np.zeros((0,) + k.shape[2:])
    return attn_fwd(q, k, v, empty, empty, scale)


def causal_prefill_bwd(q, k, v, dout, scale: float = 0.0):
    """Gradients of plain causal attention (no cartridge, nothing frozen)."""
    empty = np.zeros((0,) + np.asarray(k).shape[2:])
    dq, dk, dv, _, _ = attn_bwd(q, k, v, empty, empty, dout, scale, 0)
    return dq, dk, dv


# --------------------------------------------------------------------------
# Serving ("Semantics", serving: an empty cache takes the prefix rows in its
# own dtype, its length becomes p, decoding resumes at position p;
# "Evidence", serving parity).
# --------------------------------------------------------------------------

def round_bf16(x):
    """float32 -> bfloat16 round-to-nearest-even, returned as float64.

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit,
    then truncate the low 16 bits. NaN stays NaN (quietened).
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = (r & 0xFFFFFFFF).astype(np.uint32)
    nan = np.isnan(x32)
    r = np.where(nan, (x32.view(np.uint32) | 0x00400000) & 0xFFFF0000, r)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class DenseCache:
    """Per-sequence dense K/V rows in the cache dtype (bfloat16 values held
    as float64). No paging: the paged layout is a storage detail of the GPU
    cache, not part of what attention computes."""

    def __init__(self, n_seqs: int, n_kv_heads: int, head_dim: int):
        self.k = [np.zeros((0, n_kv_heads, head_dim)) for _ in range(n_seqs)]
        self.v = [np.zeros((0, n_kv_heads, head_dim)) for _ in range(n_seqs)]

    def seq_len(self, s: int) -> int:
        return self.k[s].shape[0]

    def append(self, s: int, k_rows, v_rows):
        """Append rows [r, Hkv, d], converted to bfloat16 (RNE)."""
        self.k[s] = np.concatenate([self.k[s], round_bf16(k_rows)], axis=0)
        self.v[s] = np.concatenate([self.v[s], round_bf16(v_rows)], axis=0)

    def write(self, s: int, k_cart, v_cart):
        """Write the whole prefix into an empty sequence; length becomes p."""
        if self.seq_len(s) != 0:
            raise ValueError("cache sequence is not empty")
        self.append(s, k_cart, v_cart)


def decode_step(cache: DenseCache, q, k_new=None, v_new=None,
                scale: float = 0.0):
    """One decode step for every sequence of ``cache``.

    q [S, Hq, d] is already rotated at position seq_len(s). If k_new/v_new
    [S, Hkv, d] are given they are appended first (so the token sees
    itself). Each query then attends over every stored row with no mask.
    Returns o [S, Hq, d] float64.
    """
    q = np.asarray(q, np.float64)
    S, Hq, d = q.shape
    if k_new is not None:
        for s in range(S):
            cache.append(s, np.asarray(k_new)[s:s + 1], np.asarray(v_new)[s:s + 1])
    if scale == 0.0:
        scale = default_scale(d)
    out = np.zeros((S, Hq, d))
    for s in range(S):
        K, V = cache.k[s], cache.v[s]
        Hkv = K.shape[1]
        g = Hq // Hkv
        for h in range(Hq):
            kv = h // g
            sc = scale * (K[:, kv, :] @ q[s, h, :])
            w = np.exp(sc - sc.max())
            out[s, h, :] = (w / w.sum()) @ V[:, kv, :]
    return out


# --------------------------------------------------------------------------
# Finite differences (the "Evidence" gradcheck procedure).
# --------------------------------------------------------------------------

def fd_grad(f, x, index_list, h: float = 1e-6):
    """Central differences of scalar f at x for the listed flat indices."""
    x = np.array(x, dtype=np.float64, copy=True)
    flat = x.reshape(-1)
    out = np.zeros(len(index_list))
    for t, idx in enumerate(index_list):
        old = flat[idx]
        flat[idx] = old + h
        fp = f(x)
        flat[idx] = old - h
        fm = f(x)
        flat[idx] = old
        out[t] = (fp - fm) / (2.0 * h)
    return out
