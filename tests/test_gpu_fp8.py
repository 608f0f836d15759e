"""Block-scaled FP8 projection weights for the decode GEMMs (pie_attach_fp8_weights).

The model is one whose projections are block-scaled FP8 (synth.fp8_block_bits:
e4m3 codes times a power-of-two scale per 128 x 128 block), so its bf16
weights are exactly the codes times their scales.  A context with the FP8
copies attached streams half the projection bytes in decode-sized calls and
must compute exactly what the same context without them computes: the
logits of every decode step are compared bit for bit.  At the tiny shape the
FP8 model is also checked against the oracle.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle.epilogue import apply
from oracle.run import Session, SynthWeights, default_numerics
from tests.parity import say
from tests.test_gpu_tiny import make_runtime

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def run_decode(rt, prompts, teach, steps):
    """Prefill every prompt, then `steps` decode steps fed the teacher tokens;
    returns the logits of every step, [steps + 1][n_seq][vocab]."""
    from paged_kv_forward_amd.runtime import Pass
    n = len(prompts)
    ws = [rt.alloc() for _ in range(n)]
    _, lg = rt.forward([Pass(ws[s], prompts[s], [len(prompts[s]) - 1], [(0, 1.0, 0)]) for s in range(n)],
                       want_logits=True)
    out = [lg]
    for k in range(steps):
        _, lg = rt.forward([Pass(ws[s], [int(teach[s][k])], [0], [(0, 1.0, 0)]) for s in range(n)],
                           want_logits=True)
        out.append(lg)
    return np.stack(out)


def test_tiny_fp8_weights_decode_equals_bf16_and_matches_oracle(torch_cuda):
    recipe = synth.WeightRecipe(synth.TINY, weight_seed=99, gain_std=0.02, fp8_blocks=True)
    shape = recipe.shape
    n, steps = 4, 6
    prompts = [synth.prompt_tokens(1, 60 + s, 24 + 5 * s, shape.vocab) for s in range(n)]
    teach = [synth.prompt_tokens(1, 70 + s, steps, shape.vocab) for s in range(n)]
    rt_bf16 = make_runtime(shape, recipe, torch_cuda)
    ref = run_decode(rt_bf16, prompts, teach, steps)
    rt_bf16.close()
    rt_fp8 = make_runtime(shape, recipe, torch_cuda, fp8=True)
    got = run_decode(rt_fp8, prompts, teach, steps)
    rt_fp8.close()
    np.testing.assert_array_equal(got, ref)
    # control: FP8 copies of another model's projections change every decode
    # step (so decode reads them) and no prefill (which keeps the bf16 weights)
    from paged_kv_forward_amd.runtime import PieRuntime, upload_weights
    wa = upload_weights(recipe, fp8=True)
    wb = upload_weights(dataclasses.replace(recipe, weight_seed=7), fp8=True)
    for la, lb in zip(wa["layers"], wb["layers"]):
        la["fp8"] = lb["fp8"]
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * 2
    rt_mix = PieRuntime(shape, wa, page_bytes * 2048, 512, 16, 64, 1024)
    mix = run_decode(rt_mix, prompts, teach, steps)
    rt_mix.close()
    np.testing.assert_array_equal(mix[0], ref[0])
    for k in range(1, steps + 1):
        assert np.max(np.abs(mix[k] - ref[k])) > 1e-2, k
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    worst = 0.0
    for s in range(n):
        sess = Session(w, num)
        seq = [prompts[s]] + [[int(t)] for t in teach[s]]
        for k, toks in enumerate(seq):
            lo = sess.step(toks)[0]
            worst = max(worst, float(np.max(np.abs(got[k][s] - lo))))
            tok, margin = apply(lo, 0)
            assert margin < 2e-2 or int(np.argmax(got[k][s])) == tok, (s, k)
    assert worst <= 2e-2, worst


def test_fp8_weights_8b_two_layers_decode_batch64_equals_bf16(torch_cuda):
    """The 8B shape cut to 2 layers, batch 64: split-K QKV / O / down, the
    56-column gate/up tiles whose lanes cross 16-row panels and 128-row scale
    blocks, all with FP8 weights, bit for bit against the bf16 weights."""
    shape = dataclasses.replace(synth.LLAMA_8B, n_layers=2)
    recipe = synth.WeightRecipe(shape, fp8_blocks=True)
    n, plen, steps = 64, 48, 3
    prompts = [synth.prompt_tokens(2, s, plen, shape.vocab) for s in range(n)]
    teach = [synth.prompt_tokens(3, s, steps, shape.vocab) for s in range(n)]
    kw = dict(max_rows=n * plen, max_seqs=n, max_readout=n, max_ctx=plen + steps + 8, pages=n * 5)
    rt_bf16 = make_runtime(shape, recipe, torch_cuda, **kw)
    ref = run_decode(rt_bf16, prompts, teach, steps)
    rt_bf16.close()
    rt_fp8 = make_runtime(shape, recipe, torch_cuda, fp8=True, **kw)
    got = run_decode(rt_fp8, prompts, teach, steps)
    rt_fp8.close()
    np.testing.assert_array_equal(got, ref)


def test_fp8_weights_70b_two_layers_e4m3_kv_decode_equals_bf16(torch_cuda):
    """The 70B shape cut to 2 layers (d_model 8192, GQA group 8, d_ffn 28672,
    e4m3 KV), batch 32: FP8 weights bit for bit against the bf16 weights."""
    shape = dataclasses.replace(synth.LLAMA_70B, n_layers=2)
    recipe = synth.WeightRecipe(shape, fp8_blocks=True)
    n, plen, steps = 32, 40, 2
    prompts = [synth.prompt_tokens(5, s, plen, shape.vocab) for s in range(n)]
    teach = [synth.prompt_tokens(6, s, steps, shape.vocab) for s in range(n)]
    kw = dict(max_rows=n * plen, max_seqs=n, max_readout=n, max_ctx=plen + steps + 8, pages=n * 5)
    rt_bf16 = make_runtime(shape, recipe, torch_cuda, **kw)
    ref = run_decode(rt_bf16, prompts, teach, steps)
    rt_bf16.close()
    rt_fp8 = make_runtime(shape, recipe, torch_cuda, fp8=True, **kw)
    got = run_decode(rt_fp8, prompts, teach, steps)
    rt_fp8.close()
    np.testing.assert_array_equal(got, ref)



def _fp8_layout_index(n, k, kc):
    """Byte of code (n, k) in the FP8 tiled layout documented in include/pie.h
    and gemm.h: 4 KiB blocks of 64 x 64 at block (n / 64, k / 64), each
    [4 panels of 16 rows][64 lanes][16 bytes], lane = (k % 32) / 8 * 16 + n % 16,
    byte = (k % 64) / 32 * 8 + k % 8."""
    r, kk = n % 64, k % 64
    return (((n // 64) * kc + k // 64) * 4096 + (r // 16) * 1024 + (((kk % 32) // 8) * 16 + r % 16) * 16
            + (kk // 32) * 8 + kk % 8)


def _rounding_inputs(n, k, seed):
    """bf16 [n][k] values the quantiser has to round: normals whose spread
    changes by row, an all-zero block, a tiny block (exponent floor), ties
    between neighbouring codes, a block maximum exactly 448 * 2^e, bf16
    subnormals, negative values that round to zero, NaN and infinities."""
    from oracle.numerics import round_bf16
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)) * np.exp(rng.uniform(-6, 6, size=(n, 1)))
    if n > 128 and k > 128:
        w[:128, 128:256] = 0.0
        w[128:256, :128] *= 1e-37
    # block (0, 0): spread 10, maximum set to 448 * 2^-2 exactly, so its scale is 2^-2
    w[:128, :128] = rng.standard_normal(w[:128, :128].shape) * 10.0
    w = round_bf16(w)
    w[0, 0] = 448.0 * 0.25
    w[0, 1:5] = np.array([1.0625, 1.1875, -1.1875, 2.0 ** -10]) * 0.25
    w[0, 5] = 2.0 ** -133          # smallest bf16 subnormal
    w[0, 6] = -2.0 ** -30           # rounds to a signed zero
    w[1, :3] = [np.nan, np.inf, -np.inf]
    assert np.nanmax(np.abs(np.where(np.isinf(w[:128, :128]), 0, w[:128, :128]))) == 112.0
    return w


@pytest.mark.parametrize("n,k", [(300, 260), (128, 128), (64, 1000), (257, 130), (16, 64)])
def test_pack_weight_fp8_rounds_like_the_oracle(torch_cuda, n, k):
    """pie_pack_weight_fp8 on matrices it must round: every code byte (in the
    documented tiled layout) and every block scale equals the oracle's
    quantiser (oracle/fp8.py), and the padding of partial blocks is zero."""
    import torch
    from oracle import fp8
    from oracle.numerics import bf16_bits
    from paged_kv_forward_amd import _native as N
    L = N.lib()
    w = _rounding_inputs(n, k, seed=n * 1000 + k)
    bits = bf16_bits(w)
    nanpos = np.isnan(w)
    bits[nanpos] = 0x7FC0
    src = torch.from_numpy(bits.view(np.int16).copy()).to("cuda")
    codes = torch.empty(L.pie_packed_weight_fp8_bytes(n, k), dtype=torch.uint8, device="cuda")
    scales = torch.empty(L.pie_fp8_scale_count(n, k), dtype=torch.float32, device="cuda")
    codes.fill_(0xA5)  # the call clears it
    st = torch.cuda.current_stream().cuda_stream
    assert L.pie_pack_weight_fp8(src.data_ptr(), codes.data_ptr(), scales.data_ptr(), n, k, st) == 0
    got_codes = codes.cpu().numpy()
    got_scales = scales.cpu().numpy().reshape(-(-n // 128), -(-k // 128))
    vals, want_bits, want_scales, _ = fp8.quantise(w)
    np.testing.assert_array_equal(got_scales.view(np.uint32), want_scales.view(np.uint32))
    kc = -(-k // 64)
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    idx = _fp8_layout_index(nn, kk, kc)
    got = got_codes[idx]
    np.testing.assert_array_equal(got, want_bits)
    pad = np.ones(got_codes.size, dtype=bool)
    pad[idx.reshape(-1)] = False
    assert not got_codes[pad].any()
    say("pack fp8 %dx%d: %d codes, %d scales, %d padding bytes match" % (n, k, got.size, got_scales.size, int(pad.sum())))
