"""Pins for oracle.model and oracle.run: closed forms, brute force, library
routines (torch.nn.functional, HF transformers' LlamaForCausalLM) and the
invariants the pages imply (incremental decode = full recompute; a forked
working set = recomputing its prefix; a chunk boundary anywhere gives the same
result)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle.epilogue import EPI_ARGMAX, apply, argmax_lowest
from oracle.model import Numerics, attention, layer_forward, rmsnorm, rope, silu
from oracle.run import Chunk, Session, SynthWeights, default_numerics, forward_chunks

RNG = np.random.default_rng(11)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    d, eps = 64, 1e-5
    g = RNG.standard_normal(d)
    for c in (0.0, 1e-3, 0.5, -7.0):
        y = np.full((1, d), c)
        np.testing.assert_allclose(rmsnorm(y, g, eps)[0], c / math.sqrt(c * c + eps) * g,
                                   rtol=1e-14, atol=0)


def test_rmsnorm_matches_torch():
    y = RNG.standard_normal((5, 96)) * 3
    g = RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(y), (96,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rmsnorm(y, g, 1e-5), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((3, 4, 16))
    np.testing.assert_array_equal(rope(x, np.zeros(3, dtype=int), 5e5), x)


def test_rope_two_dims_is_a_plane_rotation():
    # hd = 2: one pair (x0, x1) at frequency theta^0 = 1, rotated by angle p
    x = RNG.standard_normal((4, 1, 2))
    p = np.array([0, 1, 2, 37])
    r = rope(x, p, 10000.0)
    for i in range(4):
        c, s = math.cos(p[i]), math.sin(p[i])
        np.testing.assert_allclose(r[i, 0], [x[i, 0, 0] * c - x[i, 0, 1] * s,
                                             x[i, 0, 1] * c + x[i, 0, 0] * s], rtol=1e-13)


def test_rope_pairs_and_frequencies():
    # hd = 4: pairs (0,2) and (1,3); the second pair turns at theta^(-2/4)
    theta, p = 100.0, 3
    e = np.eye(4)[:, None, :]          # four unit vectors, one head
    r = rope(e, np.full(4, p), theta)
    w1 = theta ** -0.5
    np.testing.assert_allclose(r[0, 0], [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    np.testing.assert_allclose(r[1, 0], [0, math.cos(p * w1), 0, math.sin(p * w1)], atol=1e-15)
    np.testing.assert_allclose(r[2, 0], [-math.sin(p), 0, math.cos(p), 0], atol=1e-15)


def test_rope_keeps_pair_norms_and_is_relative():
    hd = 32
    q = RNG.standard_normal((1, 1, hd))
    k = RNG.standard_normal((1, 1, hd))
    for m, n in [(5, 2), (1000, 999), (8191, 17)]:
        rq = rope(q, np.array([m]), 5e5)
        rk = rope(k, np.array([n]), 5e5)
        lhs = float(np.sum(rq * rk))
        rhs = float(np.sum(rope(q, np.array([m - n]), 5e5) * k))
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs))
        half = hd // 2
        np.testing.assert_allclose(rq[0, 0, :half] ** 2 + rq[0, 0, half:] ** 2,
                                   q[0, 0, :half] ** 2 + q[0, 0, half:] ** 2, rtol=1e-12)


# ---------------------------------------------------------------- attention

def _brute_attention(q, K, V, n_ctx):
    n, nq, hd = q.shape
    nkv = K.shape[1]
    out = np.zeros_like(q)
    for i in range(n):
        for h in range(nq):
            kv = h // (nq // nkv)
            sc = []
            for j in range(n_ctx + i + 1):
                sc.append(sum(q[i, h, t] * K[j, kv, t] for t in range(hd)) / math.sqrt(hd))
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            for t in range(hd):
                out[i, h, t] = sum(w[j] * V[j, kv, t] for j in range(len(w))) / tot
    return out


@pytest.mark.parametrize("n,n_ctx", [(1, 0), (5, 0), (3, 7), (1, 19), (12, 4)])
def test_attention_brute_force(n, n_ctx):
    nq, nkv, hd = 4, 2, 8
    q = RNG.standard_normal((n, nq, hd))
    K = RNG.standard_normal((n_ctx + n, nkv, hd))
    V = RNG.standard_normal((n_ctx + n, nkv, hd))
    np.testing.assert_allclose(attention(q, K, V, n_ctx), _brute_attention(q, K, V, n_ctx),
                               rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_gqa():
    n, nq, nkv, hd = 17, 8, 2, 16
    q = RNG.standard_normal((n, nq, hd))
    K = RNG.standard_normal((n, nkv, hd))
    V = RNG.standard_normal((n, nkv, hd))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(t(q), t(K), t(V), is_causal=True, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(attention(q, K, V, 0), ref, rtol=1e-10, atol=1e-12)


def test_attention_chunk_with_context_equals_full():
    n, nq, nkv, hd = 20, 4, 1, 8
    q = RNG.standard_normal((n, nq, hd))
    K = RNG.standard_normal((n, nkv, hd))
    V = RNG.standard_normal((n, nkv, hd))
    full = attention(q, K, V, 0)
    np.testing.assert_allclose(attention(q[13:], K, V, 13), full[13:], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- SiLU

def test_silu():
    x = RNG.standard_normal(1000) * 5
    np.testing.assert_allclose(silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)
    assert silu(np.array([0.0]))[0] == 0.0
    big = np.array([30.0, 60.0])
    np.testing.assert_allclose(silu(big) / big, 1.0, rtol=1e-12)
    assert abs(silu(np.array([-60.0]))[0]) < 1e-24


# ---------------------------------------------------------------- argmax

def test_argmax_one_hot_ties_and_numpy():
    for hot in (0, 7, 4095):
        v = np.zeros(4096)
        v[hot] = 1.0
        assert apply(v, EPI_ARGMAX)[0] == hot
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0])
    assert argmax_lowest(v) == 1
    for _ in range(20):
        x = RNG.standard_normal(1000)
        assert argmax_lowest(x) == int(np.argmax(x))


# ---------------------------------------------------------------- whole forward

TINY_GAINS = synth.WeightRecipe(synth.TINY, weight_seed=99, gain_std=0.02)


def _hf_llama(recipe):
    from transformers import LlamaConfig, LlamaForCausalLM
    s = recipe.shape
    cfg = LlamaConfig(vocab_size=s.vocab, hidden_size=s.d_model, intermediate_size=s.d_ffn,
                      num_hidden_layers=s.n_layers, num_attention_heads=s.n_q_heads,
                      num_key_value_heads=s.n_kv_heads, head_dim=s.head_dim,
                      rms_norm_eps=s.rms_eps, rope_theta=s.rope_theta,
                      max_position_embeddings=4096, tie_word_embeddings=False,
                      attention_bias=False, mlp_bias=False, attn_implementation="eager")
    m = LlamaForCausalLM(cfg).to(torch.float64).eval()
    f = lambda bits: torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(f(recipe.embed_bits()))
        m.model.norm.weight.copy_(f(recipe.final_norm_bits()))
        m.lm_head.weight.copy_(f(recipe.head_bits()))
        for l in range(s.n_layers):
            lw = recipe.layer_bits(l)
            L = m.model.layers[l]
            L.input_layernorm.weight.copy_(f(lw["attn_norm"]))
            L.post_attention_layernorm.weight.copy_(f(lw["mlp_norm"]))
            L.self_attn.q_proj.weight.copy_(f(lw["q"]))
            L.self_attn.k_proj.weight.copy_(f(lw["k"]))
            L.self_attn.v_proj.weight.copy_(f(lw["v"]))
            L.self_attn.o_proj.weight.copy_(f(lw["o"]))
            L.mlp.gate_proj.weight.copy_(f(lw["gate"]))
            L.mlp.up_proj.weight.copy_(f(lw["up"]))
            L.mlp.down_proj.weight.copy_(f(lw["down"]))
    return m


def test_exact_forward_matches_hf_llama():
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    toks = synth.prompt_tokens(1, 0, 40, synth.TINY.vocab)
    num = Numerics(exact=True)
    ours = forward_chunks(w, [Chunk(toks, np.arange(40), -1, list(range(40)))], num)[0]
    hf = _hf_llama(TINY_GAINS)
    with torch.no_grad():
        ref = hf(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    err = np.max(np.abs(ours - ref))
    assert err < 1e-5, err


def test_rounded_forward_stays_close_to_exact():
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    toks = synth.prompt_tokens(1, 1, 32, synth.TINY.vocab)
    ch = [Chunk(toks, np.arange(32), -1, [31])]
    a = forward_chunks(w, ch, Numerics(exact=True))[0]
    b = forward_chunks(w, ch, default_numerics(synth.TINY))[0]
    assert np.max(np.abs(a - b)) < 5e-2          # informative: bf16 storage points


def test_incremental_decode_equals_full_recompute():
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    num = default_numerics(synth.TINY)
    toks = synth.prompt_tokens(1, 2, 24, synth.TINY.vocab)
    full = forward_chunks(w, [Chunk(toks, np.arange(24), -1, list(range(24)))], num)[0]
    sess = Session(w, num)
    inc = [sess.step(toks[:10], readout=list(range(10)))]
    for i in range(10, 24):
        inc.append(sess.step(toks[i:i + 1]))
    inc = np.concatenate(inc)
    np.testing.assert_allclose(inc, full, rtol=0, atol=1e-6)
    assert [argmax_lowest(r) for r in inc] == [argmax_lowest(r) for r in full] or \
        np.max(np.abs(inc - full)) < 1e-6


def test_chunk_boundaries_do_not_matter():
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    num = default_numerics(synth.TINY)
    toks = synth.prompt_tokens(1, 3, 30, synth.TINY.vocab)
    one = forward_chunks(w, [Chunk(toks, np.arange(30), -1, [29])], num)[0]
    cuts = [0, 7, 16, 17, 30]
    chunks = [Chunk(toks[a:b], np.arange(a, b), i - 1, [b - a - 1] if b == 30 else [])
              for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:]))]
    many = forward_chunks(w, chunks, num)[-1]
    np.testing.assert_allclose(many, one, rtol=0, atol=1e-6)


def test_fork_equals_recompute_of_prefix_plus_suffix():
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    num = default_numerics(synth.TINY)
    pre = synth.prompt_tokens(1, 4, 21, synth.TINY.vocab)
    sufs = [synth.prompt_tokens(1, 5 + b, 6, synth.TINY.vocab) for b in range(3)]
    tree = [Chunk(pre, np.arange(21), -1, [])] + \
        [Chunk(s, 21 + np.arange(6), 0, [5]) for s in sufs]
    got = forward_chunks(w, tree, num)[1:]
    for b, s in enumerate(sufs):
        whole = np.concatenate([pre, s])
        ref = forward_chunks(w, [Chunk(whole, np.arange(27), -1, [26])], num)[0]
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-6)
    # the session path: fork copies and continues independently
    sess = Session(w, num)
    sess.step(pre, readout=[])
    kid = sess.fork()
    np.testing.assert_allclose(kid.step(sufs[0]), got[0], rtol=0, atol=1e-6)


def test_wrong_positions_are_caught_by_the_invariant():
    """A plausible mistake (RoPE positions restarting at 0 in each chunk)
    breaks chunk-boundary invariance: the pin has teeth."""
    w = SynthWeights(TINY_GAINS, cache_layers=True)
    num = default_numerics(synth.TINY)
    toks = synth.prompt_tokens(1, 6, 20, synth.TINY.vocab)
    one = forward_chunks(w, [Chunk(toks, np.arange(20), -1, [19])], num)[0]
    bad = forward_chunks(w, [Chunk(toks[:12], np.arange(12), -1, []),
                             Chunk(toks[12:], np.arange(8), 0, [7])], num)[-1]
    assert np.max(np.abs(bad - one)) > 1e-2


def test_e4m3_kv_path_runs_and_stays_close_to_bf16():
    import dataclasses
    shape = dataclasses.replace(synth.TINY, kv_dtype=synth.KV_E4M3)
    w = SynthWeights(synth.WeightRecipe(shape), cache_layers=True)
    toks = synth.prompt_tokens(1, 7, 32, shape.vocab)
    ch = [Chunk(toks, np.arange(32), -1, [31])]
    e = forward_chunks(w, ch, default_numerics(shape))[0]
    b = forward_chunks(w, ch, Numerics(exact=False, kv_dtype=synth.KV_BF16))[0]
    assert 0 < np.max(np.abs(e - b)) < 0.5


# ---------------------------------------------------------------- e4m3 KV scales

def _pow2_scales(L, nkv):
    """Distinct power-of-two scales per (layer, K|V, head): 2^(5l + 3w + h - 12)."""
    s = np.empty((L, 2, nkv), dtype=np.float32)
    for l in range(L):
        for w in range(2):
            for h in range(nkv):
                s[l, w, h] = 2.0 ** (5 * l + 3 * w + h - 12)
    return s


def test_e4m3_kv_applies_the_scale_of_its_layer_kind_and_head():
    """Values that are exact codes times the right scale store losslessly;
    a K/V, head or layer mix-up changes the scale by a power of two other than
    1, which saturates 448 or flushes 2^-9 to zero.  A tie (1.0625 between
    codes 1 and 1.125) rounds to the even code."""
    L, nkv, hd = 3, 4, 8
    scales = _pow2_scales(L, nkv)
    num = Numerics(exact=False, kv_dtype=synth.KV_E4M3, kv_scales=scales)
    pattern = np.array([448.0, -448.0, 2.0 ** -9, -2.0 ** -9, 1.125, 0.0, 240.0, 1.0625])
    for l in range(L):
        for w in range(2):
            x = np.empty((5, nkv, hd))
            for h in range(nkv):
                x[:, h, :] = float(scales[l, w, h]) * pattern[None, :]
            got = num.kv(x, l, w)
            want = x.copy()
            for h in range(nkv):
                want[:, h, 7] = float(scales[l, w, h]) * 1.0  # the tie goes to the even code
            np.testing.assert_array_equal(got, want)
            # the same values under every other scale do not survive
            for l2 in range(L):
                for w2 in range(2):
                    if (l2, w2) != (l, w):
                        assert np.any(num.kv(x, l2, w2) != want)
            rolled = np.roll(x, 1, axis=1)  # heads shifted by one
            assert np.any(num.kv(rolled, l, w) != np.roll(want, 1, axis=1))


def test_e4m3_kv_scales_reach_k_and_v_separately_in_a_layer():
    """Closed forms of one layer's attention when one of K or V is scaled so
    far up that it stores as zeros: V = 0 leaves the residual unchanged by
    attention (o = 0), and K = 0 makes every score 0, so attention averages the
    visible V rows uniformly."""
    import dataclasses
    shape = dataclasses.replace(synth.TINY, kv_dtype=synth.KV_E4M3, n_layers=1)
    w = SynthWeights(synth.WeightRecipe(shape), cache_layers=True)
    lw = w.layer(0)
    n = 6
    h = w.embed_rows(synth.prompt_tokens(1, 9, n, shape.vocab)).astype(np.float64)
    empty = np.zeros((0, shape.n_kv_heads, shape.head_dim))
    huge, ok = np.float32(2.0 ** 40), np.float32(0.05)
    # V scale huge: every stored V is zero
    sv = np.array([[[ok] * shape.n_kv_heads, [huge] * shape.n_kv_heads]], dtype=np.float32)
    num = Numerics(exact=False, kv_dtype=synth.KV_E4M3, kv_scales=sv)
    _, K, V = layer_forward(lw, h, np.arange(n), empty, empty, shape, num, 0)
    assert not np.any(V) and np.any(K)
    # the attention half of the layer adds exactly nothing: compare with a
    # layer whose o projection is zero
    lw0 = dict(lw, o=np.zeros_like(lw["o"]))
    a, _, _ = layer_forward(lw, h, np.arange(n), empty, empty, shape, num, 0)
    b, _, _ = layer_forward(lw0, h, np.arange(n), empty, empty, shape, num, 0)
    np.testing.assert_array_equal(a, b)
    # K scale huge: every stored K is zero, scores are all 0, attention is the
    # running mean of the stored V rows
    sk = np.array([[[huge] * shape.n_kv_heads, [ok] * shape.n_kv_heads]], dtype=np.float32)
    num = Numerics(exact=False, kv_dtype=synth.KV_E4M3, kv_scales=sk)
    _, K, V = layer_forward(lw, h, np.arange(n), empty, empty, shape, num, 0)
    assert not np.any(K) and np.any(V)
    G = shape.n_q_heads // shape.n_kv_heads
    q = np.zeros((n, shape.n_q_heads, shape.head_dim))
    o = attention(q, K, V, 0)
    for i in range(n):
        for hh in range(shape.n_q_heads):
            np.testing.assert_allclose(o[i, hh], V[:i + 1, hh // G].mean(axis=0), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- top-2 margin

def _brute_margin(v):
    v = [float(x) for x in v]
    if len(v) < 2:
        return math.inf
    i = max(range(len(v)), key=lambda j: (v[j], -j))
    rest = v[:i] + v[i + 1:]
    return v[i] - max(rest)


def test_top2_margin_matches_sorted_brute_force_with_ties():
    from oracle.epilogue import top2_margin
    rng = np.random.default_rng(4)
    cases = [rng.standard_normal(50), np.array([1.0, 3.0, 3.0, 2.0]), np.array([5.0]),
             np.array([-2.0, -1.0]), np.array([0.0, 0.0]), rng.integers(-3, 3, size=40).astype(float),
             np.array([-np.inf, 1.0, 0.5])]
    for v in cases:
        assert top2_margin(v) == _brute_margin(v), v
    assert top2_margin(np.array([1.0, 3.0, 3.0])) == 0.0
