"""Plain CPU float64 oracle for the mask and decode variants: a sliding
window that can cut through the prefix, and a multi-token verify step behind
the serving cache.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module. It shares no code with the GPU path.

Sources (titles of the pages the method is described on):

* "Cartridges: trained KV-prefix corpus compression" (Fucina guide), section
  "gemma4 (measured)": local sliding-window layers see a served cartridge
  exactly as a real prefix -- within the window -- and one of the exact
  mechanism gates has the window cut through the prefix; section
  "Composition": the SWA layers see a composed prefix within their window
  like a single prefix of the same length.
* Same page, section "Batched self-study (measured)": speculative decoding
  verifies a span of draft tokens per stream in one pass, attention per
  stream against its own cache, greedy acceptance per row with truncating
  rewinds of the rejected rows.

Readings:

* window W >= 1: the query at position P sees the rows at positions
  P - W + 1 .. P (the W most recent positions, itself included); cartridge
  row j sits at position j, token i at p + i (the RoPE positions);
* a verify step appends its k rows to every sequence and its token t (at
  position seq_len + t) sees every stored row up to its own: the same rows
  as k single decode steps one after another.
"""

from __future__ import annotations

import numpy as np

from oracle.cartattn_oracle import DenseCache, default_scale

__all__ = ["visible_window", "attn_fwd_window", "attn_bwd_window", "causal_prefill_window",
           "verify_step"]


def visible_window(n: int, p: int, window: int):
    """Boolean [n, p + n]: row j visible to query i iff p+i-W < j <= p+i."""
    i = np.arange(n)[:, None] + p
    j = np.arange(p + n)[None, :]
    vis = j <= i
    if window > 0:
        vis = vis & (j > i - window)
    return vis


def _concat(b, kv, k_tok, v_tok, k_cart, v_cart):
    K = np.concatenate([k_cart[:, kv, :], k_tok[b, :, kv, :]], axis=0)
    V = np.concatenate([v_cart[:, kv, :], v_tok[b, :, kv, :]], axis=0)
    return K, V


def attn_fwd_window(q, k_tok, v_tok, k_cart, v_cart, window: int, scale: float = 0.0):
    """O [B, n, Hq, d] and LSE [B, Hq, n] with the window mask (window 0:
    no window, the base end-aligned causal mask)."""
    q, k_tok, v_tok, k_cart, v_cart = (np.asarray(t, np.float64)
                                       for t in (q, k_tok, v_tok, k_cart, v_cart))
    B, n, Hq, d = q.shape
    p, Hkv = k_cart.shape[0], k_tok.shape[2]
    g = Hq // Hkv
    scale = scale or default_scale(d)
    vis = visible_window(n, p, window)
    O = np.zeros((B, n, Hq, d))
    LSE = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            K, V = _concat(b, h // g, k_tok, v_tok, k_cart, v_cart)
            S = np.where(vis, scale * (q[b, :, h, :] @ K.T), -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            O[b, :, h, :] = (E / l) @ V
            LSE[b, h, :] = (m + np.log(l))[:, 0]
    return O, LSE


def attn_bwd_window(q, k_tok, v_tok, k_cart, v_cart, dout, window: int, scale: float = 0.0,
                    frozen_rows: int = 1):
    """Gradients of sum(O * dO) under the window mask: the softmax adjoint
    (D = rowsum(dO O), dS = P (dO V^T - D)), cartridge rows summed over batch
    and group heads, rows below frozen_rows exactly zero."""
    q, k_tok, v_tok, k_cart, v_cart, dout = (np.asarray(t, np.float64)
                                             for t in (q, k_tok, v_tok, k_cart, v_cart, dout))
    B, n, Hq, d = q.shape
    p, Hkv = k_cart.shape[0], k_tok.shape[2]
    g = Hq // Hkv
    scale = scale or default_scale(d)
    vis = visible_window(n, p, window)
    dq = np.zeros_like(q)
    dkt, dvt = np.zeros_like(k_tok), np.zeros_like(v_tok)
    dkc, dvc = np.zeros_like(k_cart), np.zeros_like(v_cart)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            K, V = _concat(b, kv, k_tok, v_tok, k_cart, v_cart)
            Q, dO = q[b, :, h, :], dout[b, :, h, :]
            S = np.where(vis, scale * (Q @ K.T), -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            Dr = np.sum(dO * (P @ V), axis=1, keepdims=True)
            dS = P * (dO @ V.T - Dr)
            dq[b, :, h, :] = scale * (dS @ K)
            dK = scale * (dS.T @ Q)
            dV = P.T @ dO
            dkc[:, kv] += dK[:p]
            dvc[:, kv] += dV[:p]
            dkt[b, :, kv] += dK[p:]
            dvt[b, :, kv] += dV[p:]
    dkc[:frozen_rows] = 0.0
    dvc[:frozen_rows] = 0.0
    return dq, dkt, dvt, dkc, dvc


def causal_prefill_window(q, k, v, window: int, scale: float = 0.0):
    """Plain sliding-window causal attention over T rows (no cartridge)."""
    empty = np.zeros((0,) + np.asarray(k).shape[2:])
    return attn_fwd_window(q, k, v, empty, empty, window, scale)


def verify_step(cache: DenseCache, q, k_new, v_new, scale: float = 0.0):
    """One verify step: q [S, k, Hq, d] (token t rotated at seq_len + t),
    k_new/v_new [S, k, Hkv, d] appended first; token t of sequence s attends
    over the stored rows 0 .. old_len + t. Returns o [S, k, Hq, d]."""
    q = np.asarray(q, np.float64)
    S, kq, Hq, d = q.shape
    scale = scale or default_scale(d)
    old = [cache.seq_len(s) for s in range(S)]
    for s in range(S):
        cache.append(s, np.asarray(k_new)[s], np.asarray(v_new)[s])
    out = np.zeros((S, kq, Hq, d))
    for s in range(S):
        K, V = cache.k[s], cache.v[s]
        g = Hq // K.shape[1]
        for t in range(kq):
            rows = old[s] + t + 1
            for h in range(Hq):
                sc = scale * (K[:rows, h // g, :] @ q[s, t, h, :])
                w = np.exp(sc - sc.max())
                out[s, t, h, :] = (w / w.sum()) @ V[:rows, h // g, :]
    return out
