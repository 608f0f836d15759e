"""The two fused epilogues, applied to one readout row's logits.
Test infrastructure only.

reduce_argmax (Write an inferlet; How Pie thinks, §3 Forward passes):
  the greedy token.  Ties go to the lowest index (a reading: the pages do not
  say).
gumbel_max(logits / T, seed) (How Pie thinks, §5 Epilogues):
  temperature sampling by the Gumbel-max trick: argmax_v logits_v / T + G_v
  with G_v = -ln(-ln u_v), u_v uniform, which draws v with probability
  softmax(logits / T)_v.

The decision (the argmax) is taken in float32, the precision in which the GPU
holds logits and scores; the margin (top-2 gap) is reported in float64 so a
test can tell near-ties from real disagreements.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .philox import gumbel_uniform

EPI_ARGMAX = 0
EPI_GUMBEL = 1


def argmax_lowest(values: np.ndarray):
    """Lowest index attaining the maximum (per row for a 2-D input)."""
    values = np.asarray(values)
    if values.ndim == 2:
        return np.argmax(values == values.max(axis=1, keepdims=True), axis=1)
    return int(np.flatnonzero(values == values.max())[0])


def top2_margin(values: np.ndarray) -> float:
    v = np.asarray(values, dtype=np.float64)
    if v.size < 2:
        return np.inf
    two = np.partition(v, -2)[-2:]
    return float(two[1] - two[0])


def gumbel_noise(seed, lane, vocab: int) -> np.ndarray:
    """G_v = -ln(-ln u_v) in float64 for v in [0, vocab).  `seed` may be an
    array of shape [n] (then the result is [n, vocab])."""
    seed = np.asarray(seed, dtype=np.uint64)
    v = np.arange(vocab, dtype=np.uint64)
    if seed.ndim:
        seed = seed[:, None]
    u = gumbel_uniform(seed, lane, v)
    return -np.log(-np.log(u))


def scores(logits: np.ndarray, kind: int, temperature: float, seed: int, lane: int
           ) -> Tuple[np.ndarray, np.ndarray]:
    """The values the epilogue maximises: (float32 decision values, float64 values)."""
    logits = np.asarray(logits, dtype=np.float64)
    if kind == EPI_ARGMAX:
        return logits.astype(np.float32), logits
    if kind != EPI_GUMBEL:
        raise ValueError("unknown epilogue kind %r" % kind)
    g64 = gumbel_noise(seed, lane, logits.shape[-1])
    s32 = (logits.astype(np.float32) / np.float32(temperature)).astype(np.float32)
    s32 = (s32 + g64.astype(np.float32)).astype(np.float32)
    return s32, logits / temperature + g64


def apply(logits: np.ndarray, kind: int, temperature: float = 1.0, seed: int = 0, lane: int = 0
          ) -> Tuple[int, float]:
    """(token, top-2 margin of the decision values)."""
    s32, s64 = scores(logits, kind, temperature, seed, lane)
    return argmax_lowest(s32), top2_margin(s64)
