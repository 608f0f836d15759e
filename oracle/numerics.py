"""Rounding to the storage formats of the path.  Test infrastructure only.

The pages name the formats (Write a model in Poem, §2 Deployments; Poem ops,
"Data types": bf16, e4m3) but not where values are rounded; the rounding
points used by ``oracle.model`` are a reading of this build.

Every rounding here is written from the definition of the format: find the
value's binade, take the spacing (quantum) of representable numbers in it,
and round x / quantum to the nearest integer, ties to even (numpy.rint).  A
value first goes to float32 (the precision in which the GPU holds it) and is
then quantised, so that both sides take a rounding decision from the same
precision.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")   # (2 - 2^-7) * 2^127
E4M3_MAX = 448.0                          # OCP E4M3FN: 1.75 * 2^8, no infinities


def round_f32(x) -> np.ndarray:
    """IEEE round-to-nearest-even to float32, returned as float64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _quantise(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round x to a binary format with `mant_bits` stored mantissa bits whose
    smallest normal exponent is `min_exp` (subnormals share its quantum)."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)                 # x = m * 2^e2, 0.5 <= |m| < 1
    e = np.maximum(e2 - 1, min_exp)      # binade exponent, clamped to the normal range
    q = e - mant_bits                    # exponent of the quantum
    out[fin] = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    return out


def round_bf16(x) -> np.ndarray:
    """Value -> float32 (RNE) -> bf16 (RNE); float64 array of bf16 values.

    bf16: 8 exponent bits (bias 127), 7 stored mantissa bits, so the quantum
    in binade 2^e is 2^(e-7) and the smallest normal binade is 2^-126.
    Overflow goes to +-inf as in IEEE rounding.
    """
    x32 = round_f32(x)
    r = _quantise(x32, 7, -126)
    big = np.isfinite(r) & (np.abs(r) > BF16_MAX)
    r[big] = np.copysign(np.inf, r[big])
    return r


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of values that are already bf16."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def e4m3_code_value(x32) -> np.ndarray:
    """OCP E4M3FN quantisation of float32 values, saturating: clamp to +-448,
    then round to the grid (3 stored mantissa bits, bias 7, smallest normal
    binade 2^-6, quantum 2^-9 for subnormals).  Returns the code's value."""
    x = np.clip(np.asarray(x32, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    return _quantise(x, 3, -6)


def store_e4m3(x, scale: float) -> np.ndarray:
    """Stored value of x in an e4m3 KV page with dequantisation scale s:
    s * e4m3(clamp(fp32(x) / s)), the division done in float32."""
    s32 = np.float32(scale)
    q32 = (np.asarray(x, dtype=np.float64).astype(np.float32) / s32).astype(np.float32)
    return np.float64(s32) * e4m3_code_value(q32)
