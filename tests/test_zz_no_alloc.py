"""pie_forward_static, the entry point that allocates nothing: its kernels'
scratch is the library's static device array instead of a workspace.  Checked
through the C ABI against pie_forward on identical contexts (same weights,
same passes): two calls in a row, the second smaller, at the tiny shape and at
the 8B shape cut to 2 layers with batch 64 (split-K partials, decode
attention partials, lm_head tile maxima all in the scratch); tokens equal and
logits bit for bit (the same kernels run on the same values)."""
import ctypes

import numpy as np
import pytest

import synth
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def pair(shape, recipe, max_rows, max_seqs, max_readout, max_ctx, pages):
    from paged_kv_forward_amd.runtime import PieRuntime, upload_weights
    w = upload_weights(recipe)
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * 2
    a = PieRuntime(shape, w, page_bytes * pages, max_rows, max_seqs, max_readout, max_ctx)
    b = PieRuntime(shape, w, page_bytes * pages, max_rows, max_seqs, max_readout, max_ctx, workspace=False)
    return a, b


def same(a_out, b_out, what):
    ta, la = a_out
    tb, lb = b_out
    np.testing.assert_array_equal(ta, tb)
    np.testing.assert_array_equal(la, lb)
    say("%s: %d tokens and logits equal" % (what, len(ta)))


def test_static_scratch_equals_workspace_tiny(torch_cuda):
    from paged_kv_forward_amd import _native as N
    from paged_kv_forward_amd.runtime import Pass
    recipe = synth.WeightRecipe(synth.TINY, weight_seed=99, gain_std=0.02)
    shape = recipe.shape
    a, b = pair(shape, recipe, 256, 8, 16, 512, 256)
    prompts = [synth.prompt_tokens(1, 80 + s, 20 + 3 * s, shape.vocab) for s in range(3)]
    wa = [a.alloc() for _ in range(3)]
    wb = [b.alloc() for _ in range(3)]
    epi = lambda s, k: [(1, 0.7, synth.epilogue_seed(0x77 + s, k))]
    # call 1: a 69-row prefill batch (prefill kernels)
    same(a.forward([Pass(wa[s], prompts[s], [len(prompts[s]) - 1], epi(s, 0)) for s in range(3)], want_logits=True),
         b.forward_static([Pass(wb[s], prompts[s], [len(prompts[s]) - 1], epi(s, 0)) for s in range(3)],
                          want_logits=True), "tiny prefill")
    # call 2, smaller: a decode step of two of them
    same(a.forward([Pass(wa[s], [7 + s], [0], epi(s, 1)) for s in range(2)], want_logits=True),
         b.forward_static([Pass(wb[s], [7 + s], [0], epi(s, 1)) for s in range(2)], want_logits=True),
         "tiny decode")
    # the workspace-less context serves only the static entry point
    with pytest.raises(N.PieError) as e:
        b.forward([Pass(wb[0], [1], [0], epi(0, 2))])
    assert e.value.code == N.PIE_ESTATE
    assert b.ws_info(wb[0])["len"] == len(prompts[0]) + 1
    a.close()
    b.close()


def test_static_scratch_rejects_limits_beyond_its_size(torch_cuda):
    from paged_kv_forward_amd import _native as N
    from paged_kv_forward_amd.runtime import Pass, PieRuntime, upload_weights
    recipe = synth.WeightRecipe(synth.TINY)
    shape = recipe.shape
    big = PieRuntime(shape, upload_weights(recipe), 64 << 20, 60000, 8, 16, 60000)
    assert big.ws_bytes > N.PIE_STATIC_SCRATCH_BYTES
    h = big.alloc()
    with pytest.raises(N.PieError) as e:
        big.forward_static([Pass(h, [1, 2, 3], [2], [(0, 1.0, 0)])])
    assert e.value.code == N.PIE_ENOMEM and "static scratch" in str(e.value)
    assert big.ws_info(h)["len"] == 0  # nothing changed
    big.close()
    with pytest.raises(N.PieError) as e:
        PieRuntime(shape, upload_weights(recipe), 64 << 20, 60000, 8, 16, 60000, workspace=False)
    assert e.value.code == N.PIE_ENOMEM


def test_static_scratch_equals_workspace_8b_two_layers(torch_cuda):
    from paged_kv_forward_amd.runtime import Pass
    shape = synth.first_layers(synth.LLAMA_8B, 2)
    recipe = synth.WeightRecipe(shape)
    n, plen = 64, 16
    a, b = pair(shape, recipe, 64, 64, 64, 64, n * 4)
    assert a.ws_bytes <= 96 * 1024 * 1024
    prompts = [synth.prompt_tokens(2, 300 + s, plen, shape.vocab) for s in range(n)]
    wa = [a.alloc() for _ in range(n)]
    wb = [b.alloc() for _ in range(n)]
    for s0 in range(0, n, 4):  # prefill in 64-row launches
        a.forward([Pass(wa[s], prompts[s]) for s in range(s0, s0 + 4)])
        b.forward_static([Pass(wb[s], prompts[s]) for s in range(s0, s0 + 4)])
    feed = synth.prompt_tokens(2, 400, n, shape.vocab)
    # call 1: a 64-row decode step (split-K projections, decode attention)
    same(a.forward([Pass(wa[s], [int(feed[s])], [0], [(0, 1.0, 0)]) for s in range(n)], want_logits=True),
         b.forward_static([Pass(wb[s], [int(feed[s])], [0], [(0, 1.0, 0)]) for s in range(n)], want_logits=True),
         "8b decode 64")
    # call 2, smaller: 5 rows, Gumbel-max
    same(a.forward([Pass(wa[s], [int(feed[s]) ^ 1], [0], [(1, 0.7, 99 + s)]) for s in range(5)], want_logits=True),
         b.forward_static([Pass(wb[s], [int(feed[s]) ^ 1], [0], [(1, 0.7, 99 + s)]) for s in range(5)],
                          want_logits=True), "8b decode 5")
    a.close()
    b.close()
