"""Pins of the oracle's block-scaled FP8 quantiser (oracle/fp8.py) against
things other than itself: torch's float8_e4m3fn decoding of all 256 codes and
its cast (a library routine), the nearest code found by brute force over the
whole code table, the block scale found by searching exponents, and exact
cases (ties, the 448 boundary, all-zero and tiny blocks, NaN and infinity)."""
import numpy as np
import torch

from oracle import fp8
from oracle.numerics import round_bf16

TABLE = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
FINITE = np.isfinite(TABLE)


def bf16(x):
    return round_bf16(np.asarray(x, dtype=np.float64))


def test_code_bits_invert_torch_decoding_of_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = fp8.code_bits(TABLE)
    np.testing.assert_array_equal(got[FINITE], codes[FINITE])
    # NaN maps to a NaN code (0x7f, or 0xff when the NaN carries a sign bit)
    assert got[0x7F] in (0x7F, 0xFF) and got[0xFF] in (0x7F, 0xFF)


def brute_nearest(x):
    """Nearest finite code value to x by search; ties to the even code."""
    v = TABLE[FINITE]
    c = np.arange(256)[FINITE]
    d = np.abs(v[None, :] - x[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    out = np.empty(len(x))
    for i in range(len(x)):
        cs = c[cand[i]]
        vs = v[cand[i]]
        if len(cs) > 1:  # a tie between two neighbours: the even mantissa wins
            vs = vs[(cs & 1) == 0]  # (+0 and -0 are both even and equal)
        out[i] = vs[0]
    return out


def brute_exponent(amax):
    if amax == 0:
        return fp8.MIN_EXP
    for e in range(-200, 200):
        if amax <= 448.0 * 2.0 ** e:
            return max(e, fp8.MIN_EXP)
    raise AssertionError


def test_quantise_matches_brute_force_on_random_blocks():
    rng = np.random.default_rng(11)
    w = bf16(rng.standard_normal((300, 260)) * np.exp(rng.uniform(-8, 8, size=(300, 1))))
    w[:128, 128:256] = 0.0                              # an all-zero block
    w[128:256, :128] *= 1e-36                           # a tiny block (exponent clamp)
    w = bf16(w)
    vals, bits, scales, exps = fp8.quantise(w)
    for i in range(0, 300, 128):
        for j in range(0, 260, 128):
            blk = w[i:i + 128, j:j + 128]
            e = brute_exponent(float(np.abs(blk).max()))
            assert exps[i // 128, j // 128] == e
            assert scales[i // 128, j // 128] == np.float32(2.0 ** e)
            x = (blk / 2.0 ** e).reshape(-1)
            idx = rng.choice(x.size, size=min(400, x.size), replace=False)
            np.testing.assert_array_equal(vals[i:i + 128, j:j + 128].reshape(-1)[idx], brute_nearest(x[idx]))
    # every code times its scale is a bf16 number
    deq = fp8.dequantise(vals, scales)
    np.testing.assert_array_equal(round_bf16(deq), deq)


def test_quantise_agrees_with_torch_cast():
    rng = np.random.default_rng(3)
    w = bf16(rng.standard_normal((256, 384)) * 0.02)
    w[5, 7] = 3.0
    vals, bits, scales, _ = fp8.quantise(w)
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
    t = torch.from_numpy(np.clip(w / s, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(t.view(torch.uint8).numpy(), bits)
    np.testing.assert_array_equal(t.float().numpy().astype(np.float64), vals)


def test_exact_cases():
    # amax exactly 448 * 2^3: e = 3, and the maximum maps to the largest code
    w = np.zeros((128, 128))
    w[0, 0] = 448.0 * 8
    w[0, 1] = -448.0 * 8
    # ties at scale 2^3: 1.0625 lies halfway between codes 1.0 and 1.125 (even: 1.0),
    # 1.1875 halfway between 1.125 and 1.25 (even: 1.25); 2^-10 between 0 and 2^-9 (even: 0)
    w[1, 0], w[1, 1], w[1, 2], w[1, 3] = 1.0625 * 8, 1.1875 * 8, -1.1875 * 8, 2.0 ** -10 * 8
    vals, bits, scales, exps = fp8.quantise(w)
    assert exps[0, 0] == 3
    assert bits[0, 0] == 0x7E and bits[0, 1] == 0xFE
    assert vals[1, 0] == 1.0 and vals[1, 1] == 1.25 and vals[1, 2] == -1.25 and vals[1, 3] == 0.0
    assert bits[1, 3] == 0x00
    # just above 448 * 2^3 (the next bf16 number): e = 4
    w[0, 0] = bf16(448.0 * 8 * (1 + 2.0 ** -7))
    assert fp8.quantise(w)[3][0, 0] == 4
    # an all-zero block: scale 2^MIN_EXP, every code 0
    v, b, s, e = fp8.quantise(np.zeros((130, 3)))
    assert (b == 0).all() and (e == fp8.MIN_EXP).all()
    # a tiny block keeps exponent MIN_EXP and rounds on the bf16-subnormal grid
    t = np.full((4, 4), 2.0 ** -130)
    v, b, s, e = fp8.quantise(t)
    assert e[0, 0] == fp8.MIN_EXP and (v == 2.0 ** -6).all() and (b == 0x08).all()
    # NaN is left out of the maximum and keeps the NaN code; infinity saturates
    u = np.ones((8, 8))
    u[0, 0], u[0, 1], u[0, 2] = np.nan, np.inf, -np.inf
    v, b, s, e = fp8.quantise(u)
    assert e[0, 0] == fp8.block_exponent(1.0) == -8
    assert b[0, 0] == 0x7F and b[0, 1] == 0x7E and b[0, 2] == 0xFE
    # negative values that round to zero keep their sign bit
    z = np.ones((2, 2))
    z[1, 1] = -2.0 ** -20
    assert fp8.quantise(z)[1][1, 1] == 0x80


def test_e4m3_nan_stays_nan_and_torch_agrees():
    from oracle.numerics import e4m3_code_value
    assert np.isnan(e4m3_code_value(np.float32(np.nan)))
    assert np.isnan(torch.tensor([float("nan")]).to(torch.float8_e4m3fn).float().item())
