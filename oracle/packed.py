"""Plain CPU float64 oracle for packed segments behind one cartridge: several
variable-length token segments packed back to back into one token tensor,
each attending causally over itself behind the shared prefix.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module. It shares no code with the GPU path.

Source: "Cartridges: trained KV-prefix corpus compression" (Fucina guide),
section "Deliberate divergences from the reference": packing runs a group of
conversations as contiguous segments of one forward -- RoPE restarts per
segment, attention runs per segment (the reference's block mask), and the
gradients flow through the usual backward, packed gradients equal to
sequential ones; section "Batched self-study (measured)": the packed
training step is one forward/backward for the group; section "Deliberate
divergences from the paper": the packed forward shares one prefix across
its segments.

Readings: segment s occupies packed rows
cu[s] .. cu[s+1]-1 (cu = running sum of the lengths); its token t sits at
RoPE position p + t; the cartridge gradient is the sum over segments.
"""

from __future__ import annotations

import numpy as np

from oracle.cartattn_oracle import attn_bwd, attn_fwd

__all__ = ["seg_offsets", "packed_positions", "attn_fwd_packed", "attn_bwd_packed"]


def seg_offsets(seg_lens):
    """cu[0] = 0, cu[s+1] = cu[s] + seg_lens[s]."""
    return np.concatenate([[0], np.cumsum(np.asarray(seg_lens, dtype=np.int64))])


def packed_positions(seg_lens, p: int):
    """RoPE position of every packed row: p + (row - cu[segment])."""
    return np.concatenate([p + np.arange(int(n), dtype=np.int64) for n in seg_lens])


def attn_fwd_packed(q, k_tok, v_tok, k_cart, v_cart, seg_lens, scale: float = 0.0):
    """q [T, Hq, d], k_tok/v_tok [T, Hkv, d] packed. Each segment is the
    single-sequence attention behind the shared cartridge.
    Returns (O [T, Hq, d], list of LSE [Hq, len_s])."""
    cu = seg_offsets(seg_lens)
    O = np.zeros(np.asarray(q).shape)
    lses = []
    for s in range(len(seg_lens)):
        r = slice(int(cu[s]), int(cu[s + 1]))
        o, lse = attn_fwd(np.asarray(q)[None, r], np.asarray(k_tok)[None, r],
                          np.asarray(v_tok)[None, r], k_cart, v_cart, scale)
        O[r] = o[0]
        lses.append(lse[0])
    return O, lses


def attn_bwd_packed(q, k_tok, v_tok, k_cart, v_cart, dout, seg_lens, scale: float = 0.0,
                    frozen_rows: int = 1):
    """Gradients of sum(O * dO) over all segments: token gradients per
    segment, the cartridge gradient summed over the segments (rows below
    frozen_rows exactly zero)."""
    cu = seg_offsets(seg_lens)
    q = np.asarray(q, np.float64)
    dq = np.zeros_like(q)
    dkt = np.zeros(np.asarray(k_tok).shape)
    dvt = np.zeros(np.asarray(v_tok).shape)
    dkc = np.zeros(np.asarray(k_cart).shape)
    dvc = np.zeros(np.asarray(v_cart).shape)
    for s in range(len(seg_lens)):
        r = slice(int(cu[s]), int(cu[s + 1]))
        g = attn_bwd(q[None, r], np.asarray(k_tok)[None, r], np.asarray(v_tok)[None, r],
                     k_cart, v_cart, np.asarray(dout)[None, r], scale, frozen_rows=0)
        dq[r], dkt[r], dvt[r] = g[0][0], g[1][0], g[2][0]
        dkc += g[3]
        dvc += g[4]
    dkc[:frozen_rows] = 0.0
    dvc[:frozen_rows] = 0.0
    return dq, dkt, dvt, dkc, dvc
