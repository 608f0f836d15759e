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

