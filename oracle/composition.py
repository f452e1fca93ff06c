"""Plain CPU float64 oracle for composed cartridges: a prefix made of several
independently trained parts, each with its own frozen sink rows.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module. It shares no code with the GPU path.

Source: "Cartridges: trained KV-prefix corpus compression" (Fucina guide),
section "Composition": parts compose by concatenation -- part 0's rows, then
part 1's, and so on -- and the real tokens sit at RoPE positions equal to the
total number of composed rows; every part keeps the rotations it was trained
at (overlapping nominal positions across parts are harmless, attention only
takes dot products against the frozen post-RoPE keys); the composed prefix is
one concatenation per layer, so the attention backward routes gradients into
every part's trainable rows while every part's sink stays frozen; serving
writes the parts in order into an empty cache with the append primitive.

Readings: each part freezes its own first
``frozen[i]`` rows (the base method's frozen_prefix, per part); the tokens'
first position is the composed length P = sum of the parts' rows.
"""

from __future__ import annotations

import numpy as np

from oracle.cartattn_oracle import attn_bwd, attn_fwd

__all__ = ["composed_p", "compose", "frozen_mask", "attn_fwd_composed", "attn_bwd_composed"]


def composed_p(rows) -> int:
    """Total composed rows: the tokens' first RoPE position."""
    return int(sum(int(r) for r in rows))


def compose(parts_k, parts_v):
    """The concatenation of the parts' rows, part 0 first: [P, Hkv, d]."""
    return (np.concatenate([np.asarray(k, np.float64) for k in parts_k], axis=0),
            np.concatenate([np.asarray(v, np.float64) for v in parts_v], axis=0))


def frozen_mask(rows, frozen):
    """Boolean [P]: True on each part's own first frozen[i] rows."""
    mask = []
    for r, f in zip(rows, frozen):
        m = np.zeros(int(r), dtype=bool)
        m[: int(f)] = True
        mask.append(m)
    return np.concatenate(mask) if mask else np.zeros(0, dtype=bool)


def attn_fwd_composed(q, k_tok, v_tok, parts_k, parts_v, scale: float = 0.0):
    """O and LSE of the attention over concat(parts..., tokens)."""
    kc, vc = compose(parts_k, parts_v)
    return attn_fwd(q, k_tok, v_tok, kc, vc, scale)


def attn_bwd_composed(q, k_tok, v_tok, parts_k, parts_v, dout, frozen, scale: float = 0.0):
    """Gradients through the composed concat.

    Returns (dq, dk_tok, dv_tok, dk_parts, dv_parts): the per-part cartridge
    gradients (lists, part order) with each part's frozen rows exactly zero.
    """
    kc, vc = compose(parts_k, parts_v)
    dq, dkt, dvt, dkc, dvc = attn_bwd(q, k_tok, v_tok, kc, vc, dout, scale, frozen_rows=0)
    rows = [np.asarray(k).shape[0] for k in parts_k]
    mask = frozen_mask(rows, frozen)
    dkc[mask] = 0.0
    dvc[mask] = 0.0
    cuts = np.cumsum(rows)[:-1]
    return dq, dkt, dvt, np.split(dkc, cuts, axis=0), np.split(dvc, cuts, axis=0)
