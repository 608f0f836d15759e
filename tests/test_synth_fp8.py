"""The block-scaled FP8 weights a FP8 model is drawn with (synth.fp8_block_bits):
every 128 x 128 block is e4m3 codes times 2^e, e the least integer with
max |w| <= 448 * 2^e, and each value is the nearest such code (by brute force
over all 256 codes on a sample)."""
import numpy as np
import torch

import synth


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_fp8_blocks_are_codes_times_power_of_two_scales():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((300, 200)) * 0.02).astype(np.float32)
    w[0, 0] = 0.9  # one block with a much larger amax
    w[150:, 150:] = 0.0  # an all-zero block region
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    q = _f32(synth.fp8_block_bits(bits))
    src = _f32(bits)
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    codes = codes[np.isfinite(codes)]
    for r0 in range(0, 300, 128):
        for c0 in range(0, 200, 128):
            blk, sblk = q[r0:r0 + 128, c0:c0 + 128], src[r0:r0 + 128, c0:c0 + 128]
            amax = float(np.abs(sblk).max())
            if amax == 0.0:
                assert not np.any(blk)
                continue
            e = int(np.ceil(np.log2(amax / 448.0)))
            e += int(amax > 448.0 * 2.0 ** e)
            e -= int(amax <= 448.0 * 2.0 ** (e - 1))
            assert amax <= 448.0 * 2.0 ** e and amax > 448.0 * 2.0 ** (e - 1)
            scaled = blk / 2.0 ** e
            assert np.all(np.isin(scaled, codes))  # exact codes
            # nearest code to each source value (sample of 64 entries)
            sv = (sblk / 2.0 ** e).reshape(-1)[::257][:64]
            got = scaled.reshape(-1)[::257][:64]
            d = np.abs(codes[None, :] - sv[:, None])
            best = d.min(axis=1)
            assert np.all(np.abs(got - sv) <= best + 1e-12)


def test_fp8_recipe_touches_projections_and_head_only():
    r8 = synth.WeightRecipe(synth.TINY, fp8_blocks=True)
    r = synth.WeightRecipe(synth.TINY)
    assert np.array_equal(r8.tensor_bits("embed", (64, 256)), r.tensor_bits("embed", (64, 256)))
    assert np.array_equal(r8.tensor_bits("layers.0.attn_norm", (256,)), r.tensor_bits("layers.0.attn_norm", (256,)))
    assert not np.array_equal(r8.tensor_bits("head", (64, 256)), r.tensor_bits("head", (64, 256)))
    assert not np.array_equal(r8.tensor_bits("layers.0.q", (256, 256)), r.tensor_bits("layers.0.q", (256, 256)))
