"""Pins for oracle.numerics: the bf16 and e4m3 roundings against PyTorch's own
casts (library routines), and exhaustive code round trips."""
import numpy as np
import pytest
import torch

from oracle.numerics import (BF16_MAX, E4M3_MAX, bf16_bits, e4m3_code_value, round_bf16,
                             round_f32, store_e4m3)


def _edge_f32():
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 1.0, 1e3, 1e30)]
    # exact ties between two bf16 neighbours: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**31, 5000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    vals.append(ties.view(np.float32))
    # subnormals and the largest finite floats
    vals.append(np.array([1e-40, -1e-40, 1.5e-45, 3.4e38, -3.4e38, 3.3895e38, 0.0, -0.0],
                         dtype=np.float32))
    return np.concatenate(vals)


def test_bf16_matches_torch_cast():
    x = _edge_f32()
    ours = round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_from_double_goes_through_float32():
    # a double just above a bf16 tie: float32 rounding lands on the tie first,
    # then ties-to-even decides (the kernel's precision takes the decision)
    tie = np.float64(1.0 + 2.0 ** -8)               # midway between 1 and 1 + 2^-7
    x = tie + 2.0 ** -40                             # rounds to the tie in float32
    assert round_f32(x) == tie
    assert round_bf16(x) == 1.0                      # tie -> even mantissa


def test_bf16_overflow_and_specials():
    assert np.isinf(round_bf16(np.float64(3.4e38)))[()] or round_bf16(3.4e38) == np.inf
    assert round_bf16(BF16_MAX) == BF16_MAX
    assert np.isnan(round_bf16(np.nan))
    assert round_bf16(-np.inf) == -np.inf


def test_bf16_bits_roundtrip_all_finite_codes():
    codes = np.arange(1 << 16, dtype=np.uint32)
    vals = (codes << 16).view(np.float32)
    fin = np.isfinite(vals)
    r = round_bf16(vals[fin])
    np.testing.assert_array_equal(r, vals[fin].astype(np.float64))
    np.testing.assert_array_equal(bf16_bits(r), codes[fin].astype(np.uint16))


def test_e4m3_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (0.01, 1.0, 30.0, 1000.0)])
    x = np.concatenate([x, [0.0, -0.0, 448.0, -448.0, 464.0, 1e9, -1e9, 2.0 ** -10, 2.0 ** -9,
                            3 * 2.0 ** -10, 2.0 ** -6 + 2.0 ** -10]]).astype(np.float32)
    ours = e4m3_code_value(x)
    clamped = torch.from_numpy(x).clamp(-E4M3_MAX, E4M3_MAX)
    ref = clamped.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_all_256_codes_roundtrip():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    fin = np.isfinite(vals)
    assert fin.sum() == 254                       # 0x7f and 0xff are NaN, no infinities
    np.testing.assert_array_equal(e4m3_code_value(vals[fin].astype(np.float32)), vals[fin])
    assert vals[fin].max() == 448.0 and np.min(np.abs(vals[fin][vals[fin] != 0])) == 2.0 ** -9


def test_store_e4m3_saturates_and_scales():
    s = 0.0123
    x = np.array([1e6, -1e6, 0.0, 447.0 * s, 3.0 * s])
    st = store_e4m3(x, s)
    s32 = np.float64(np.float32(s))
    assert st[0] == 448.0 * s32 and st[1] == -448.0 * s32 and st[2] == 0.0
    assert st[4] == 3.0 * s32
