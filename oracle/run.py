"""Driving the oracle over whole workloads.  Test infrastructure only.

A workload is a set of *chunks*: runs of new tokens of one sequence, each with
the chunk it continues (its parent), so that a chunk's context is the tokens of
all its ancestors, root first.  This covers one whole prompt (one chunk), a
prompt fed in pieces or token by token (a chain), and working sets forked off
a shared frozen prefix (a tree: "ws.fork() ... shares the frozen prefix",
How Pie thinks, §4 Working sets).  Every chunk is recomputed from its own
tokens with contiguous KV; nothing is shared between chunks except the K/V
values of ancestors, which by definition do not depend on descendants.

``forward_chunks`` goes layer-major (all chunks through layer l, then l+1), so
each layer's weights are drawn once, which keeps the 8B and 70B shapes within
host memory.  ``Session`` goes token-major with a per-layer KV cache for
free-running decode loops at small shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import synth
from .model import Numerics, head_logits, layer_forward


class SynthWeights:
    """Weights of a ``synth.WeightRecipe`` as float32 arrays (exact bf16 values)."""

    def __init__(self, recipe: "synth.WeightRecipe", cache_layers: bool = False):
        self.recipe = recipe
        self.shape = recipe.shape
        self._cache_layers = cache_layers
        self._layers: Dict[int, Dict[str, np.ndarray]] = {}
        self._head = None
        self._final = None

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        if l in self._layers:
            return self._layers[l]
        lw = {k: synth.bf16_bits_to_f32(v) for k, v in self.recipe.layer_bits(l).items()}
        if self._cache_layers:
            self._layers[l] = lw
        return lw

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        tokens = np.asarray(tokens, dtype=np.int64)
        uniq, inv = np.unique(tokens, return_inverse=True)
        rows = synth.bf16_bits_to_f32(self.recipe.embed_rows_bits(uniq))
        return rows[inv.reshape(-1)]

    def final_norm(self) -> np.ndarray:
        if self._final is None:
            self._final = synth.bf16_bits_to_f32(self.recipe.final_norm_bits())
        return self._final

    def head(self) -> np.ndarray:
        if self._head is None:
            self._head = synth.bf16_bits_to_f32(self.recipe.head_bits())
        return self._head

    def drop_head(self):
        self._head = None


def default_numerics(shape, exact: bool = False, kv_scales=None) -> Numerics:
    return Numerics(exact=exact, kv_dtype=shape.kv_dtype,
                    kv_scales=kv_scales if kv_scales is not None else
                    (synth.kv_scales(shape) if shape.kv_dtype == synth.KV_E4M3 else None))


@dataclass
class Chunk:
    tokens: np.ndarray
    positions: np.ndarray
    parent: int = -1                  # index of the chunk this one continues, -1 = none
    readout: Sequence[int] = ()       # row indices inside this chunk to read out


def _ancestors(chunks: List[Chunk], i: int) -> List[int]:
    out = []
    p = chunks[i].parent
    while p >= 0:
        if p >= i:
            raise ValueError("a chunk's parent must come before it")
        out.append(p)
        p = chunks[p].parent
    return out[::-1]


def forward_chunks(weights: SynthWeights, chunks: List[Chunk], num: Numerics,
                   want_hidden: bool = False) -> List[np.ndarray]:
    """Logits [len(readout), V] (float64 holding float32 values) for every chunk."""
    shape = weights.shape
    anc = [_ancestors(chunks, i) for i in range(len(chunks))]
    h = [weights.embed_rows(c.tokens).astype(np.float64) for c in chunks]
    empty = np.zeros((0, shape.n_kv_heads, shape.head_dim))
    for l in range(shape.n_layers):
        lw = weights.layer(l)
        Ks: List[np.ndarray] = [None] * len(chunks)
        Vs: List[np.ndarray] = [None] * len(chunks)
        for i, c in enumerate(chunks):
            if anc[i]:
                K_ctx = np.concatenate([Ks[a] for a in anc[i]], axis=0)
                V_ctx = np.concatenate([Vs[a] for a in anc[i]], axis=0)
            else:
                K_ctx, V_ctx = empty, empty
            h[i], Ks[i], Vs[i] = layer_forward(lw, h[i], np.asarray(c.positions), K_ctx, V_ctx,
                                               shape, num, l)
        del lw
    out = []
    for i, c in enumerate(chunks):
        ro = list(c.readout)
        if not ro:
            out.append(np.zeros((0, shape.vocab)))
            continue
        out.append(head_logits(h[i][ro], weights.final_norm(), weights.head(), shape, num))
    if want_hidden:
        return out, h
    return out


class Session:
    """One sequence, token-major, with contiguous per-layer KV.  ``fork`` copies
    the KV arrays (the oracle has no pages to share)."""

    def __init__(self, weights: SynthWeights, num: Numerics):
        self.w = weights
        self.num = num
        s = weights.shape
        self.K = [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)]
        self.V = [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(s.n_layers)]
        self.tokens: List[int] = []

    def __len__(self):
        return len(self.tokens)

    def fork(self, keep: Optional[int] = None) -> "Session":
        n = len(self) if keep is None else keep
        c = Session.__new__(Session)
        c.w, c.num = self.w, self.num
        c.K = [k[:n].copy() for k in self.K]
        c.V = [v[:n].copy() for v in self.V]
        c.tokens = list(self.tokens[:n])
        return c

    def step(self, tokens, positions=None, readout: Sequence[int] = (-1,)) -> np.ndarray:
        tokens = np.asarray(tokens, dtype=np.int64)
        if positions is None:
            positions = len(self) + np.arange(len(tokens))
        s = self.w.shape
        h = self.w.embed_rows(tokens).astype(np.float64)
        for l in range(s.n_layers):
            h, Kn, Vn = layer_forward(self.w.layer(l), h, np.asarray(positions), self.K[l],
                                      self.V[l], s, self.num, l)
            self.K[l] = np.concatenate([self.K[l], Kn], axis=0)
            self.V[l] = np.concatenate([self.V[l], Vn], axis=0)
        self.tokens.extend(int(t) for t in tokens)
        ro = [r % len(tokens) for r in readout]
        if not ro:
            return np.zeros((0, s.vocab))
        return head_logits(h[ro], self.w.final_norm(), self.w.head(), s, self.num)
