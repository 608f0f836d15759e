"""Block-scaled FP8 weights: the quantiser, written from the format's definition.
Test infrastructure only.

The pages list a block-scaled FP8 weight dtype, e4m3tile128a8 ("Write a model
in Poem", section 2 Deployments; "Poem ops", Data types) without defining the
blocking.  Reading taken (the HIP path documents the same one at its
boundary):

  * blocks of 128 x 128 entries of the [out][in] matrix, ragged at the edges;
  * one power-of-two scale 2^e per block, e the least integer with
    max |w| <= 448 * 2^e over the block's finite entries (0 for a block with
    no non-zero finite entry), and never below MIN_EXP = -124, so that every
    code times its scale is a bf16 number (the smallest non-zero code is 2^-9);
  * the code of w is OCP E4M3FN round-to-nearest-even of w / 2^e, saturating
    at +-448; NaN keeps the NaN code.

Codes are returned both as values (float64) and as their 8-bit patterns
(sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
the subnormals m * 2^-9; 0x7f / 0xff is NaN).
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, e4m3_code_value

BLOCK = 128
MIN_EXP = -124


def block_exponent(amax: float) -> int:
    """Least integer e with amax <= 448 * 2^e (MIN_EXP at least; MIN_EXP for amax 0)."""
    if not amax > 0.0:
        return MIN_EXP
    e = int(np.floor(np.log2(amax / E4M3_MAX)))
    # the float log2 may be off by one at exact powers: settle by comparison
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(e, MIN_EXP)


def code_bits(values) -> np.ndarray:
    """8-bit E4M3FN patterns of values that lie on the e4m3 grid (or are NaN);
    the sign bit is the value's own (so -0.0 gives 0x80)."""
    v = np.asarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    nan = np.isnan(v)
    sub = ~nan & (a < 2.0 ** -6)
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.uint8)         # m * 2^-9, m = 0..7
    nrm = ~nan & ~sub
    _, e2 = np.frexp(a[nrm])                                         # a = f * 2^e2, 0.5 <= f < 1
    e = e2 - 1                                                       # binade 2^e, e in -6 .. 8
    m = np.rint(a[nrm] / 2.0 ** e * 8.0).astype(np.int64) - 8        # 3 mantissa bits
    out[nrm] = ((e + 7) << 3 | m).astype(np.uint8)
    out[nan] = 0x7F
    return out | sign


def quantise(w) -> tuple:
    """w: [n][k] weights (float).  Returns (code values [n][k] float64,
    code bits [n][k] uint8, scales [ceil(n/128)][ceil(k/128)] float32, e)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    nb, kb = -(-n // BLOCK), -(-k // BLOCK)
    exps = np.zeros((nb, kb), dtype=np.int64)
    vals = np.empty_like(w)
    for i in range(nb):
        for j in range(kb):
            blk = w[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK]
            fin = np.abs(blk[np.isfinite(blk)])
            e = block_exponent(float(fin.max()) if fin.size else 0.0)
            exps[i, j] = e
            # w / 2^e is exact in float64 for every bf16 w and e >= MIN_EXP
            vals[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK] = \
                e4m3_code_value(np.ldexp(blk, -e).astype(np.float32))
    scales = np.ldexp(1.0, exps).astype(np.float32)
    return vals, code_bits(vals), scales, exps


def dequantise(vals, scales) -> np.ndarray:
    """Weights the codes stand for: code value * its block's scale (float64)."""
    vals = np.asarray(vals, dtype=np.float64)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), BLOCK, 0), BLOCK, 1)
    return vals * s[:vals.shape[0], :vals.shape[1]]
