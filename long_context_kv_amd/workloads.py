"""Seeded synthetic inputs for the cartridge-attention workloads.

This module only draws random numbers and fixes shapes; it holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may take their
inputs from it. Every tensor is drawn on the CPU with a seeded
``torch.Generator`` in a fixed order, as float32 N(0, 1), and then cast to its
storage dtype (bfloat16 by round-to-nearest-even, which is torch's cast).

The pages measure on a paper dataset and on real model weights, neither of
which is available; these N(0, 1) tensors at the layer shapes of the Qwen3
family stand in for them.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

THETA = 1.0e6          # RoPE base of the Qwen3 family
FROZEN_ROWS = 1        # the attention-sink row is frozen by default
PAGE_SIZE = 16         # rows per page of the serving cache


@dataclasses.dataclass(frozen=True)
class TrainShape:
    """One attention layer of a cartridge training step."""
    name: str
    batch: int
    q_seq: int
    p: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tok_dtype: torch.dtype
    cart_dtype: torch.dtype
    seed: int
    layers: int = 1
    frozen_rows: int = FROZEN_ROWS

    @property
    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the end-aligned mask keeps."""
        n, p = self.q_seq, self.p
        return self.batch * self.n_q_heads * (n * p + n * (n + 1) // 2)

    def fwd_flop(self) -> float:
        return 4.0 * self.head_dim * self.visible_pairs * self.layers

    def bwd_flop(self) -> float:
        return 8.0 * self.head_dim * self.visible_pairs * self.layers


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    """A batch of sequences decoding one token behind a written prefix."""
    name: str
    n_seqs: int
    p: int
    max_generated: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    seed: int


# The five workloads: a tiny float32 reference-mode layer, three Qwen3-shaped
# training layers and a serving decode batch.
TINY = TrainShape("tiny-f32", 1, 16, 8, 4, 2, 64, torch.float32, torch.float32, 1)
QWEN3_0_6B = TrainShape("qwen3-0.6b-layer", 1, 1024, 2048, 16, 8, 128,
                        torch.bfloat16, torch.float32, 2)
QWEN3_8B = TrainShape("qwen3-8b-layer", 4, 2048, 4096, 32, 8, 128,
                      torch.bfloat16, torch.float32, 3)
DECODE = DecodeShape("serving-decode", 64, 4096, 1024, 32, 8, 128, PAGE_SIZE, 4)
LONG = TrainShape("long-cartridge-28l", 1, 4096, 16384, 16, 8, 128,
                  torch.bfloat16, torch.float32, 500, layers=28)


def _randn(g: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def train_inputs(shape: TrainShape, seed: Optional[int] = None,
                 q_scale: float = 1.0) -> Dict[str, torch.Tensor]:
    """CPU tensors q, k_tok, v_tok, k_cart, v_cart, dout for one layer.

    Drawn in that order from ``seed`` (default: the shape's seed). ``q_scale``
    multiplies the float32 draw of q before the cast (used to sharpen the
    softmax in stress tests).
    """
    g = torch.Generator().manual_seed(shape.seed if seed is None else seed)
    B, n, p = shape.batch, shape.q_seq, shape.p
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    q = (torch.randn(B, n, Hq, d, generator=g) * q_scale).to(shape.tok_dtype)
    k_tok = _randn(g, (B, n, Hkv, d), shape.tok_dtype)
    v_tok = _randn(g, (B, n, Hkv, d), shape.tok_dtype)
    k_cart = _randn(g, (p, Hkv, d), shape.cart_dtype)
    v_cart = _randn(g, (p, Hkv, d), shape.cart_dtype)
    dout = _randn(g, (B, n, Hq, d), shape.tok_dtype)
    return dict(q=q, k_tok=k_tok, v_tok=v_tok, k_cart=k_cart, v_cart=v_cart,
                dout=dout)


def prefill_raw(T: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                seed: int, dtype: torch.dtype = torch.float32, batch: int = 1):
    """Unrotated q, k, v [batch, T, H, d] for the prefill-equivalence check:
    the first p rows become the cartridge after rotation at 0..p-1."""
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (batch, T, n_q_heads, head_dim), dtype)
    k = _randn(g, (batch, T, n_kv_heads, head_dim), dtype)
    v = _randn(g, (batch, T, n_kv_heads, head_dim), dtype)
    dout = _randn(g, (batch, T, n_q_heads, head_dim), dtype)
    return q, k, v, dout


@dataclasses.dataclass
class DecodeInputs:
    generated: List[int]          # rows generated after the prefix, per seq
    k_cart: torch.Tensor          # [p, Hkv, d] float32, shared artifact
    v_cart: torch.Tensor
    k_gen: List[torch.Tensor]     # per seq [generated[s], Hkv, d] bfloat16
    v_gen: List[torch.Tensor]
    q: torch.Tensor               # [S, Hq, d] bfloat16
    page_perm: torch.Tensor       # physical page order, int32
    max_pages_per_seq: int
    n_pages: int


def decode_inputs(shape: DecodeShape, n_seqs: Optional[int] = None,
                  p: Optional[int] = None,
                  max_generated: Optional[int] = None,
                  seed: Optional[int] = None) -> DecodeInputs:
    """Seeded serving inputs, drawn in this order: generated lengths
    U{0..max_generated}; one shared cartridge K/V (float32); each sequence's
    generated K/V (bfloat16); q (bfloat16); a random physical page order."""
    S = shape.n_seqs if n_seqs is None else n_seqs
    p = shape.p if p is None else p
    G = shape.max_generated if max_generated is None else max_generated
    Hq, Hkv, d, P = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.page_size
    g = torch.Generator().manual_seed(shape.seed if seed is None else seed)
    generated = torch.randint(0, G + 1, (S,), generator=g).tolist()
    k_cart = _randn(g, (p, Hkv, d), torch.float32)
    v_cart = _randn(g, (p, Hkv, d), torch.float32)
    k_gen, v_gen = [], []
    for s in range(S):
        k_gen.append(_randn(g, (generated[s], Hkv, d), torch.bfloat16))
        v_gen.append(_randn(g, (generated[s], Hkv, d), torch.bfloat16))
    q = _randn(g, (S, Hq, d), torch.bfloat16)
    # room for the prefix, the generated rows and one appended step
    max_pages = (p + G + 1 + P - 1) // P
    n_pages = S * max_pages
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    return DecodeInputs(generated, k_cart, v_cart, k_gen, v_gen, q, perm,
                        max_pages, n_pages)


@dataclasses.dataclass
class RaggedDecodeInputs:
    k_cart: List[torch.Tensor]    # per seq [prefix[s], Hkv, d] float32
    v_cart: List[torch.Tensor]
    k_gen: List[torch.Tensor]     # per seq [generated[s], Hkv, d] bfloat16
    v_gen: List[torch.Tensor]
    q: torch.Tensor               # [S, Hq, d] bfloat16
    k_new: torch.Tensor           # [S, Hkv, d] bfloat16, one appended row each
    v_new: torch.Tensor
    page_perm: torch.Tensor       # physical page order, int32, S * max_pages
    n_pages: int


def decode_inputs_ragged(prefix: List[int], generated: List[int], n_q_heads: int,
                         n_kv_heads: int, head_dim: int, max_pages: int,
                         seed: int) -> RaggedDecodeInputs:
    """Serving inputs with a given prefix and generated length per sequence,
    drawn in this order: per sequence its prefix K/V (float32) and generated
    K/V (bfloat16); q; the appended row's K/V; a random physical page order."""
    g = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d = len(prefix), n_q_heads, n_kv_heads, head_dim
    kc, vc, kg, vg = [], [], [], []
    for s in range(S):
        kc.append(_randn(g, (prefix[s], Hkv, d), torch.float32))
        vc.append(_randn(g, (prefix[s], Hkv, d), torch.float32))
        kg.append(_randn(g, (generated[s], Hkv, d), torch.bfloat16))
        vg.append(_randn(g, (generated[s], Hkv, d), torch.bfloat16))
    q = _randn(g, (S, Hq, d), torch.bfloat16)
    k_new = _randn(g, (S, Hkv, d), torch.bfloat16)
    v_new = _randn(g, (S, Hkv, d), torch.bfloat16)
    n_pages = S * max_pages
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    return RaggedDecodeInputs(kc, vc, kg, vg, q, k_new, v_new, perm, n_pages)


SHAPES = {1: TINY, 2: QWEN3_0_6B, 3: QWEN3_8B, 4: DECODE, 5: LONG}
