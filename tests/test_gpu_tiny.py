"""GPU parity at the tiny 2-layer shape (every row checked) through the C ABI.

The oracle runs first; GPU decode passes are then fed the oracle's tokens
(teacher forcing by the oracle), so every GPU readout is compared with the
oracle on identical inputs.  A free-running loop is checked too, up to the
first near-tie.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle.epilogue import apply
from oracle.run import Chunk, Session, SynthWeights, default_numerics, forward_chunks
from tests.parity import Report, say, tau_for, twin_bounds

pytestmark = pytest.mark.gpu

N_SEQ, PROMPT, STEPS = 4, 32, 8


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def make_runtime(shape, recipe, torch_cuda, max_rows=512, max_seqs=16, max_readout=64, max_ctx=1024,
                 pages=2048, fp8=False):
    from paged_kv_forward_amd.runtime import PieRuntime, upload_weights
    w = upload_weights(recipe, fp8=fp8)
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * (
        1 if shape.kv_dtype == synth.KV_E4M3 else 2)
    return PieRuntime(shape, w, page_bytes * pages, max_rows, max_seqs, max_readout, max_ctx)


RECIPES = {
    "gains1": synth.WeightRecipe(synth.TINY),
    "gains_spread": synth.WeightRecipe(synth.TINY, weight_seed=99, gain_std=0.02),
}


def oracle_greedy(recipe, prompts, steps, kinds, temps, seeds_fn):
    """Oracle free-running loop per sequence: returns per seq list of (token, margin, logits)."""
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(recipe.shape)
    out = []
    for s, pr in enumerate(prompts):
        sess = Session(w, num)
        lg = sess.step(pr)[0]
        rows = []
        for k in range(steps + 1):
            tok, margin = apply(lg, kinds[s], temps[s], seeds_fn(s, k), 0)
            rows.append((tok, margin, lg))
            if k < steps:
                lg = sess.step([tok])[0]
        out.append(rows)
    return out


@pytest.mark.parametrize("rname", list(RECIPES))
@pytest.mark.parametrize("kind", [0, 1])
def test_tiny_prefill_then_decode_teacher_forced(torch_cuda, rname, kind):
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES[rname]
    shape = recipe.shape
    prompts = [synth.prompt_tokens(1, s, PROMPT, shape.vocab) for s in range(N_SEQ)]
    kinds = [kind] * N_SEQ
    temps = [0.7] * N_SEQ
    seed = lambda s, k: synth.epilogue_seed(0x1000 + s, k)
    say("tiny %s kind=%d: oracle" % (rname, kind))
    ref = oracle_greedy(recipe, prompts, STEPS, kinds, temps, seed)
    say("tiny %s kind=%d: gpu" % (rname, kind))
    rt = make_runtime(shape, recipe, torch_cuda)
    ws = [rt.alloc() for _ in range(N_SEQ)]
    rep = Report()
    toks, logits = rt.forward([Pass(ws[s], prompts[s], [PROMPT - 1], [(kind, 0.7, seed(s, 0))])
                               for s in range(N_SEQ)], want_logits=True)
    for s in range(N_SEQ):
        t, m, lg = ref[s][0]
        rep.add(toks[s], t, m, tau_for(kind, 0.7), logits[s], lg, ("prefill", s))
    for k in range(1, STEPS + 1):
        feed = [ref[s][k - 1][0] for s in range(N_SEQ)]
        toks, logits = rt.forward([Pass(ws[s], [feed[s]], [0], [(kind, 0.7, seed(s, k))])
                                   for s in range(N_SEQ)], want_logits=True)
        for s in range(N_SEQ):
            t, m, lg = ref[s][k]
            rep.add(toks[s], t, m, tau_for(kind, 0.7), logits[s], lg, ("decode", k, s))
    rep.check()
    for s in range(N_SEQ):
        info = rt.ws_info(ws[s])
        assert info["len"] == PROMPT + STEPS and info["frozen_len"] == PROMPT + STEPS
    rt.close()


def test_tiny_free_running_agrees_until_a_near_tie(torch_cuda):
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains1"]
    shape = recipe.shape
    prompts = [synth.prompt_tokens(1, s, PROMPT, shape.vocab) for s in range(N_SEQ)]
    ref = oracle_greedy(recipe, prompts, STEPS, [0] * N_SEQ, [1.0] * N_SEQ, lambda s, k: 0)
    rt = make_runtime(shape, recipe, torch_cuda)
    ws = [rt.alloc() for _ in range(N_SEQ)]
    toks, _ = rt.forward([Pass(ws[s], prompts[s], [PROMPT - 1], [(0, 1.0, 0)]) for s in range(N_SEQ)])
    gen = [[int(t)] for t in toks]
    for k in range(STEPS):
        toks, _ = rt.forward([Pass(ws[s], [gen[s][-1]], [0], [(0, 1.0, 0)]) for s in range(N_SEQ)])
        for s in range(N_SEQ):
            gen[s].append(int(toks[s]))
    agree = 0
    for s in range(N_SEQ):
        for k in range(STEPS + 1):
            t, m, _ = ref[s][k]
            if gen[s][k] != t:
                assert m < 2e-2, (s, k, gen[s][k], t, m)
                break
            agree += 1
    say("free-running: %d of %d steps agree before any near-tie" % (agree, N_SEQ * (STEPS + 1)))


def test_tiny_determinism_and_batch_invariance(torch_cuda):
    """Batch invariance ("How Pie thinks", Batching: a pass's result does not
    depend on what it is packed with).  Every kernel computes a row from that
    row's inputs alone, so while a batch stays within the decode-sized
    kernels (at most 64 rows) a pass alone is bit-identical to the same pass
    in the batch.  A batch of more rows runs the prefill kernels, whose
    accumulation order differs: then alone and packed both match the oracle
    (2e-2).  Two identical runs are bit-identical."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    w_or = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    for lens in ((14, 17, 20), (20, 23, 26)):
        prompts = [synth.prompt_tokens(1, 10 + s, lens[s], shape.vocab) for s in range(3)]
        outs = []
        for rep in range(2):
            rt = make_runtime(shape, recipe, torch_cuda)
            ws = [rt.alloc() for _ in range(3)]
            _, lg = rt.forward([Pass(ws[s], prompts[s], [len(prompts[s]) - 1], [(0, 1, 0)])
                                for s in range(3)], want_logits=True)
            outs.append(lg)
            # each pass alone, in a fresh working set
            alone = []
            for s in range(3):
                w = rt.alloc()
                _, l1 = rt.forward([Pass(w, prompts[s], [len(prompts[s]) - 1], [(0, 1, 0)])],
                                   want_logits=True)
                alone.append(l1[0])
            alone = np.stack(alone)
            if sum(lens) <= 64:
                np.testing.assert_array_equal(alone, lg)
            else:
                ref = forward_chunks(w_or, [Chunk(p, np.arange(len(p)), -1, [len(p) - 1]) for p in prompts], num)
                ref = np.stack([r[0] for r in ref])
                err_b, err_a = float(np.max(np.abs(lg - ref))), float(np.max(np.abs(alone - ref)))
                say("batch of %d rows vs oracle %.4g, alone vs oracle %.4g, batch vs alone %.4g" %
                    (sum(lens), err_b, err_a, float(np.max(np.abs(lg - alone)))))
                assert err_b <= 2e-2 and err_a <= 2e-2
            rt.close()
        np.testing.assert_array_equal(outs[0], outs[1])


def test_tiny_fork_partial_page_and_mixed_launch(torch_cuda):
    """Prefix of 21 tokens (a partly filled page), forked 3 ways; suffixes and a
    decode row of another sequence share one launch.  Compared with the
    oracle's tree of chunks; no KV bytes copied, shared pages kept."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    pre = synth.prompt_tokens(1, 20, 21, shape.vocab)
    sufs = [synth.prompt_tokens(1, 21 + b, 5 + 7 * b, shape.vocab) for b in range(3)]
    other = synth.prompt_tokens(1, 30, 40, shape.vocab)
    nxt = int(synth.prompt_tokens(1, 31, 1, shape.vocab)[0])
    rt = make_runtime(shape, recipe, torch_cuda)
    p = rt.alloc()
    o = rt.alloc()
    rt.forward([Pass(p, pre, [], []), Pass(o, other, [], [])])
    st0 = rt.pool_stats()
    kids = [rt.fork(p) for _ in range(3)]
    st1 = rt.pool_stats()
    assert st1["pages_ever_allocated"] == st0["pages_ever_allocated"]
    parent_pages = rt.ws_info(p)["pages"]
    for k in kids:
        np.testing.assert_array_equal(rt.ws_info(k)["pages"], parent_pages)
    passes = [Pass(kids[b], sufs[b], [len(sufs[b]) - 1], [(1, 0.7, 77 + b)]) for b in range(3)]
    passes.append(Pass(o, [nxt], [0], [(0, 1.0, 0)]))
    toks, logits = rt.forward(passes, want_logits=True)
    for b, k in enumerate(kids):
        np.testing.assert_array_equal(rt.ws_info(k)["pages"][:len(parent_pages)], parent_pages)
    assert rt.pool_stats()["kv_bytes_copied"] == 0
    # oracle
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    tree = [Chunk(pre, np.arange(21), -1, [])]
    tree += [Chunk(s, 21 + np.arange(len(s)), 0, [len(s) - 1]) for s in sufs]
    tree += [Chunk(other, np.arange(40), -1, []), Chunk(np.array([nxt]), np.array([40]), 4, [0])]
    ref = forward_chunks(w, tree, num)
    rep = Report()
    for b in range(3):
        t, m = apply(ref[1 + b][0], 1, 0.7, 77 + b, 0)
        rep.add(toks[b], t, m, tau_for(1, 0.7), logits[b], ref[1 + b][0], ("fork", b))
    t, m = apply(ref[5][0], 0)
    rep.add(toks[3], t, m, tau_for(0, 1), logits[3], ref[5][0], ("decode-in-mix",))
    rep.check()
    rt.close()


def test_tiny_e4m3_kv(torch_cuda):
    from paged_kv_forward_amd.runtime import Pass
    shape = dataclasses.replace(synth.TINY, kv_dtype=synth.KV_E4M3)
    recipe = synth.WeightRecipe(shape, weight_seed=5)
    prompts = [synth.prompt_tokens(1, 40 + s, PROMPT, shape.vocab) for s in range(N_SEQ)]
    ref = oracle_greedy(recipe, prompts, 4, [0] * N_SEQ, [1.0] * N_SEQ, lambda s, k: 0)
    rt = make_runtime(shape, recipe, torch_cuda)
    ws = [rt.alloc() for _ in range(N_SEQ)]
    rep = Report()
    toks, lg = rt.forward([Pass(ws[s], prompts[s], [PROMPT - 1], [(0, 1, 0)]) for s in range(N_SEQ)],
                          want_logits=True)
    for s in range(N_SEQ):
        rep.add(toks[s], ref[s][0][0], ref[s][0][1], 2e-2, lg[s], ref[s][0][2])
    for k in range(1, 5):
        toks, lg = rt.forward([Pass(ws[s], [ref[s][k - 1][0]], [0], [(0, 1, 0)]) for s in range(N_SEQ)],
                              want_logits=True)
        for s in range(N_SEQ):
            rep.add(toks[s], ref[s][k][0], ref[s][k][1], 2e-2, lg[s], ref[s][k][2])
    rep.check()
    rt.close()


def test_device_philox_matches_oracle(torch_cuda):
    from oracle.philox import philox4x32_10
    rt = make_runtime(synth.TINY, RECIPES["gains1"], torch_cuda)
    for seed, lane, v0 in [(0, 0, 0), (0xDEADBEEF12345678, 3, 1000), (2**64 - 1, 77, 2**32 - 5000)]:
        got = rt.philox(seed, lane, v0, 4096)
        v = (np.arange(4096, dtype=np.uint64) + np.uint64(v0)) & np.uint64(0xFFFFFFFF)
        ref = philox4x32_10(v, lane, 0, 0, seed & 0xFFFFFFFF, seed >> 32)[0]
        np.testing.assert_array_equal(got, ref)
    rt.close()


def test_graph_replays_match_direct_launches(torch_cuda, monkeypatch):
    """The same decode loop with launch graphs (captured on the second call of a
    shape, replayed after) and without: every step's logits bitwise equal."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    prompts = [synth.prompt_tokens(1, 50 + s, 24 + s, shape.vocab) for s in range(3)]
    feeds = [synth.teacher_tokens(1, s, 6, shape.vocab) for s in range(3)]
    runs = []
    for graphs in ("0", "1"):
        monkeypatch.setenv("PIE_GRAPHS", graphs)
        rt = make_runtime(shape, recipe, torch_cuda)
        ws = [rt.alloc() for _ in range(3)]
        out = []
        _, lg = rt.forward([Pass(ws[s], prompts[s], [len(prompts[s]) - 1], [(0, 1, 0)]) for s in range(3)],
                           want_logits=True)
        out.append(lg)
        dev = torch_cuda.empty((3, shape.vocab), dtype=torch_cuda.float32, device="cuda")
        for k in range(6):
            rt.forward([Pass(ws[s], [int(feeds[s][k])], [0], [(1, 0.7, 99 + k)]) for s in range(3)],
                       logits_out=dev)
            torch_cuda.cuda.synchronize()
            out.append(dev.cpu().numpy().copy())
        runs.append(out)
        rt.close()
    for a, b in zip(*runs):
        np.testing.assert_array_equal(a, b)


def packed_reference(w):
    """The tiled weight layout as include/pie.h describes it, built with numpy
    from the row-major [n][k] matrix: zero padding to multiples of 64, 64 x 64
    blocks in (row block, column block) order, each block as
    [4 panels of 16 rows][2 halves of 32 columns][4 groups of 8][16 rows][8]."""
    n, k = w.shape
    np_, kp = -(-n // 64) * 64, -(-k // 64) * 64
    pad = np.zeros((np_, kp), dtype=w.dtype)
    pad[:n, :k] = w
    b = pad.reshape(np_ // 64, 4, 16, kp // 64, 2, 4, 8)  # [rb][panel][row][cb][half][group][8]
    return b.transpose(0, 3, 1, 4, 5, 2, 6).reshape(-1)


@pytest.mark.parametrize("n,k", [(64, 64), (200, 136), (688, 256), (128, 4096 + 8)])
def test_pack_weight_layout(torch_cuda, n, k):
    from paged_kv_forward_amd import _native as N
    rng = np.random.default_rng(n * 7 + k)
    w = rng.integers(0, 1 << 16, size=(n, k), dtype=np.uint16)
    src = torch_cuda.from_numpy(w.view(np.int16)).to("cuda")
    nbytes = N.lib().pie_packed_weight_bytes(n, k)
    assert nbytes == (-(-n // 64) * 64) * (-(-k // 64) * 64) * 2
    dst = torch_cuda.full((nbytes // 2,), -1, dtype=torch_cuda.int16, device="cuda")
    N.check(N.lib().pie_pack_weight(src.data_ptr(), dst.data_ptr(), n, k, None))
    got = dst.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, packed_reference(w))
    # overlapping buffers are refused
    assert N.lib().pie_pack_weight(dst.data_ptr(), dst.data_ptr(), n, k, None) == N.PIE_EINVAL


def test_tiny_readout_lanes_positions_and_rollback(torch_cuda):
    """Several readout rows per pass (Gumbel lanes 0..2, unordered), explicit
    RoPE positions with a gap, a single-token first pass, and a writable
    buffer rolled back with pie_truncate before new tokens are appended."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    rt = make_runtime(shape, recipe, torch_cuda)
    rep = Report()
    a, b = rt.alloc(), rt.alloc()
    toks_a = synth.prompt_tokens(1, 70, 20, shape.vocab)
    pos_a = list(range(5, 15)) + list(range(115, 125))        # a gap of 100 positions
    ro_a = [19, 3, 10]
    epi_a = [(1, 0.7, 777), (1, 0.7, 777), (1, 0.7, 777)]     # lanes 0, 1, 2 of one seed
    tok_b = [int(synth.prompt_tokens(1, 71, 1, shape.vocab)[0])]  # a first pass of one token
    toks, lg = rt.forward([Pass(a, toks_a, ro_a, epi_a, positions=pos_a),
                           Pass(b, tok_b, [0], [(0, 1.0, 0)])], want_logits=True)
    sa, sb = Session(w, num), Session(w, num)
    ref_a = sa.step(toks_a, positions=pos_a, readout=ro_a)
    ref_b = sb.step(tok_b)
    for j in range(3):
        t, m = apply(ref_a[j], 1, 0.7, 777, j)
        rep.add(toks[j], t, m, tau_for(1, 0.7), lg[j], ref_a[j], ("lane", j))
    t, m = apply(ref_b[0], 0)
    rep.add(toks[3], t, m, tau_for(0, 1.0), lg[3], ref_b[0], ("single", 0))
    # uncommitted draft of 6 tokens, read out, then rolled back
    draft = synth.prompt_tokens(1, 72, 6, shape.vocab)
    rt.forward([Pass(a, draft, [5], [(0, 1.0, 0)], positions=list(range(125, 131)), commit=False)])
    info = rt.ws_info(a)
    assert info["len"] == 26 and info["frozen_len"] == 20
    rt.truncate(a, 20)
    assert rt.ws_info(a)["len"] == 20
    new = synth.prompt_tokens(1, 73, 3, shape.vocab)
    toks, lg = rt.forward([Pass(a, new, [0, 2], [(0, 1.0, 0), (1, 1.0, 5)], positions=[125, 126, 127])],
                          want_logits=True)
    ref = sa.step(new, positions=[125, 126, 127], readout=[0, 2])
    t, m = apply(ref[0], 0)
    rep.add(toks[0], t, m, tau_for(0, 1.0), lg[0], ref[0], ("after rollback", 0))
    t, m = apply(ref[1], 1, 1.0, 5, 1)
    rep.add(toks[1], t, m, tau_for(1, 1.0), lg[1], ref[1], ("after rollback", 2))
    rep.check()
    rt.close()


def test_tiny_async_loop_carried_decode(torch_cuda):
    """pie_decode_async: each step reads its tokens from the previous step's
    device output, nothing returns to the host until the end.  Every step's
    tokens and logits equal the synchronous pie_forward loop's, bit for bit,
    for argmax and for Gumbel-max with a fresh seed per step; the greedy
    trajectory agrees with the oracle's free-running loop up to a near-tie."""
    torch = torch_cuda
    recipe = RECIPES["gains1"]
    shape = recipe.shape
    prompts = [synth.prompt_tokens(1, s, PROMPT, shape.vocab) for s in range(N_SEQ)]
    ref = oracle_greedy(recipe, prompts, STEPS, [0] * N_SEQ, [1.0] * N_SEQ, lambda s, k: 0)
    rt = make_runtime(shape, recipe, torch_cuda)
    for kind, temp in [(0, 1.0), (1, 0.7)]:
        seeds = lambda k: np.array([synth.epilogue_seed(0x5EED0000 + s, k) for s in range(N_SEQ)], dtype=np.uint64)
        ws_sync = np.array([rt.alloc() for _ in range(N_SEQ)], dtype=np.uint64)
        ws_async = np.array([rt.alloc() for _ in range(N_SEQ)], dtype=np.uint64)
        first = None
        for ws in (ws_sync, ws_async):
            from paged_kv_forward_amd.runtime import Pass
            toks, _ = rt.forward([Pass(int(ws[s]), prompts[s], [PROMPT - 1], [(0, 1.0, 0)]) for s in range(N_SEQ)])
            first = toks if first is None else first
            assert list(toks) == list(first)
        # synchronous loop
        sync_toks, sync_lg = [], []
        cur = np.array(first, dtype=np.int32)
        lg = torch.empty((N_SEQ, shape.vocab), dtype=torch.float32, device="cuda")
        for k in range(STEPS):
            cur = rt.decode_step(ws_sync, cur, kind=kind, temperature=temp, seed=seeds(k), logits_out=lg)
            sync_toks.append(cur.copy())
            sync_lg.append(lg.cpu().numpy())
        # loop-carried: one device buffer is both input and output of every step
        tok_dev = torch.tensor(np.array(first, dtype=np.int32), device="cuda")
        hist = torch.empty((STEPS, N_SEQ), dtype=torch.int32, device="cuda")
        lgs = torch.empty((STEPS, N_SEQ, shape.vocab), dtype=torch.float32, device="cuda")
        for k in range(STEPS):
            rt.decode_async(ws_async, tok_dev, tok_dev, kind=kind, temperature=temp, seed=seeds(k),
                            logits_out=lgs[k])
            hist[k].copy_(tok_dev)  # same stream as the library: runs after the step
            rt.sync()
        a_toks = hist.cpu().numpy()
        for k in range(STEPS):
            np.testing.assert_array_equal(a_toks[k], sync_toks[k])
            np.testing.assert_array_equal(lgs[k].cpu().numpy(), sync_lg[k])
        for s in range(N_SEQ):
            assert rt.ws_info(int(ws_async[s]))["len"] == PROMPT + STEPS
        if kind == 0:
            gen = np.concatenate([np.array(first)[None, :], a_toks], axis=0)
            for s in range(N_SEQ):
                for k in range(STEPS + 1):
                    t, m, _ = ref[s][k]
                    if gen[k][s] != t:
                        assert m < 2e-2, (s, k, gen[k][s], t, m)
                        break
    rt.close()


def test_tiny_async_steps_enqueued_back_to_back(torch_cuda):
    """Steps enqueued without any host wait in between (more than the staging
    ring holds) give the synchronous loop's tokens; the only wait is at the end."""
    torch = torch_cuda
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    from paged_kv_forward_amd.runtime import Pass
    prompts = [synth.prompt_tokens(1, 20 + s, PROMPT + s, shape.vocab) for s in range(N_SEQ)]
    rt = make_runtime(shape, recipe, torch_cuda)
    steps = 12
    ws_a = np.array([rt.alloc() for _ in range(N_SEQ)], dtype=np.uint64)
    ws_b = np.array([rt.alloc() for _ in range(N_SEQ)], dtype=np.uint64)
    firsts = []
    for ws in (ws_a, ws_b):
        toks, _ = rt.forward([Pass(int(ws[s]), prompts[s], [len(prompts[s]) - 1], [(0, 1.0, 0)])
                              for s in range(N_SEQ)])
        firsts.append(np.array(toks, dtype=np.int32))
    cur = firsts[0]
    sync_toks = []
    for k in range(steps):
        cur = rt.decode_step(ws_a, cur)
        sync_toks.append(cur.copy())
    bufs = torch.empty((steps + 1, N_SEQ), dtype=torch.int32, device="cuda")
    bufs[0].copy_(torch.tensor(firsts[1], device="cuda"))
    torch.cuda.synchronize()
    for k in range(steps):
        rt.decode_async(ws_b, bufs[k], bufs[k + 1])
    rt.sync()
    got = bufs.cpu().numpy()[1:]
    np.testing.assert_array_equal(got, np.stack(sync_toks))
    rt.close()


def test_tiny_async_out_of_range_device_token(torch_cuda):
    """Loop-carried token ids are never checked on the host.  An id outside
    [0, vocab) (the -1 of an all-NaN logits row, or any stray value) embeds as
    a zero row: two working sets with the same prompt fed -1 and vocab + 7 give
    bit-identical logits and a valid token, and a third fed a real id differs."""
    torch = torch_cuda
    recipe = RECIPES["gains1"]
    shape = recipe.shape
    from paged_kv_forward_amd.runtime import Pass
    prompt = synth.prompt_tokens(1, 40, PROMPT, shape.vocab)
    rt = make_runtime(shape, recipe, torch_cuda)
    ws = np.array([rt.alloc() for _ in range(3)], dtype=np.uint64)
    toks, _ = rt.forward([Pass(int(w), prompt, [PROMPT - 1], [(0, 1.0, 0)]) for w in ws])
    tok_in = torch.tensor([-1, shape.vocab + 7, int(toks[0])], dtype=torch.int32, device="cuda")
    tok_out = torch.empty(3, dtype=torch.int32, device="cuda")
    lg = torch.empty((3, shape.vocab), dtype=torch.float32, device="cuda")
    rt.decode_async(ws, tok_in, tok_out, logits_out=lg)
    rt.sync()
    out, lgs = tok_out.cpu().numpy(), lg.cpu().numpy()
    assert np.all(np.isfinite(lgs))
    np.testing.assert_array_equal(lgs[0], lgs[1])
    assert out[0] == out[1] and 0 <= out[0] < shape.vocab
    assert not np.array_equal(lgs[0], lgs[2])
    rt.close()


def test_tiny_timed_attention_repeats_change_nothing(torch_cuda):
    """With decode attention timed and pie_profile_repeat(4), each decode
    attention launch runs four times back to back: the decode step's logits
    are bit-identical to an untimed step on an identical working set, and the
    class counts four launches per layer."""
    recipe = RECIPES["gains1"]
    shape = recipe.shape
    from paged_kv_forward_amd.runtime import Pass
    prompt = synth.prompt_tokens(2, 40, PROMPT, shape.vocab)
    rt = make_runtime(shape, recipe, torch_cuda)
    a, b = rt.alloc(), rt.alloc()
    toks, _ = rt.forward([Pass(w, prompt, [PROMPT - 1], [(0, 1.0, 0)]) for w in (a, b)])
    nxt = [int(toks[0])]
    _, la = rt.forward([Pass(a, nxt, [0], [(0, 1.0, 0)])], want_logits=True)
    rt.profile_repeat(4)
    rt.profile_enable(["attn_decode"])
    _, lb = rt.forward([Pass(b, nxt, [0], [(0, 1.0, 0)])], want_logits=True)
    prof = rt.profile_read()
    rt.profile_enable([])
    rt.profile_repeat(1)
    np.testing.assert_array_equal(la, lb)
    ms, n = prof["attn_decode"]
    assert n == 4 * shape.n_layers and ms > 0
    rt.close()


def test_tiny_prefix_lookup_reuses_pages_exactly(torch_cuda):
    """A request that starts with another request's committed prefix gets the
    prefix's pages through pie_prefix_lookup and runs only its own tokens: its
    readout equals a from-scratch run of the whole sequence (same kernels on
    the same values) and the oracle's, and no page is allocated for the
    shared part."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    rt = make_runtime(shape, recipe, torch_cuda)
    pre = synth.prompt_tokens(1, 40, 40, shape.vocab)
    tail = synth.prompt_tokens(1, 41, 10, shape.vocab)
    full = np.concatenate([pre[:32], tail])
    a = rt.alloc()
    rt.forward([Pass(a, pre, [39], [(0, 1.0, 0)])])
    st0 = rt.pool_stats()
    b, k = rt.prefix_lookup(full)
    assert k == 32
    assert list(rt.ws_info(b)["pages"]) == list(rt.ws_info(a)["pages"][:2])
    tb, lb = rt.forward([Pass(b, full[32:], [9], [(0, 1.0, 0)])], want_logits=True)
    assert rt.pool_stats()["pages_ever_allocated"] == st0["pages_ever_allocated"] + 1  # b's own tail page
    c = rt.alloc()
    tc, lc = rt.forward([Pass(c, full, [41], [(0, 1.0, 0)])], want_logits=True)
    assert int(tb[0]) == int(tc[0])
    np.testing.assert_allclose(lb, lc, rtol=0, atol=1e-5)
    w = SynthWeights(recipe, cache_layers=True)
    ref = Session(w, default_numerics(shape)).step(list(full))[0]
    err = float(np.max(np.abs(lb[0] - ref)))
    say("prefix reuse: max|dlogit| vs oracle %.4f" % err)
    assert err <= 2e-2
    rt.close()


@pytest.mark.parametrize("d_ffn", [688, 704])
@pytest.mark.parametrize("lens", [(150, 150), (600,), (257, 64)])
def test_tiny_large_prefill_tiles_with_ragged_edges(torch_cuda, lens, d_ffn):
    """Prefill launches of 256 rows or more use the 256 x 256 GEMM tiles: at the
    tiny shape their row and column edges are ragged (300, 600 and 321 rows;
    gate/up width 688 = 5 x 128 + 48 or 704), and the others' K (256) is a
    multiple of 64 (tiles loaded straight into LDS).  The down projection's K
    is 688, not a multiple of 64 (register-staged tile), or 704 = 11 x 64: an
    odd number of K stages, which the straight-to-LDS loop, run in pairs of
    stages, finishes with a stage of zeros.  Last-row logits of every
    sequence against the oracle."""
    from paged_kv_forward_amd.runtime import Pass
    base = RECIPES["gains_spread"]
    recipe = dataclasses.replace(base, shape=dataclasses.replace(base.shape, d_ffn=d_ffn))
    shape = recipe.shape
    rt = make_runtime(shape, recipe, torch_cuda, max_rows=1024)
    prompts = [synth.prompt_tokens(1, 60 + i, n, shape.vocab) for i, n in enumerate(lens)]
    ws = [rt.alloc() for _ in prompts]
    toks, lg = rt.forward([Pass(ws[i], prompts[i], [len(prompts[i]) - 1], [(0, 1.0, 0)])
                           for i in range(len(prompts))], want_logits=True)
    w = SynthWeights(recipe, cache_layers=True)
    rep = Report()
    for i, pr in enumerate(prompts):
        ref = Session(w, default_numerics(shape)).step(list(pr))[0]
        tok, margin = apply(ref, 0, 1.0, 0, 0)
        rep.add(toks[i], tok, margin, tau_for(0, 1.0), lg[i], ref, tag=("prefill", len(pr)))
    rep.check(max_excluded_frac=1.0, min_compared=0)  # one or two rows: the logits carry the check
    rt.close()


def test_tiny_long_decode_sequence_and_skewed_batch(torch_cuda):
    """One decode sequence with 8200 tokens of context, alone and packed with
    15 short ones: its attention is cut into more pieces than a short batch
    would take, and every piece must reach the merge (at most 64 per
    sequence).  Logits and tokens against the oracle."""
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains1"]
    shape = recipe.shape
    long_len, n_short, short_len = 8200, 15, 16
    rt = make_runtime(shape, recipe, torch_cuda, max_rows=8300, max_seqs=16, max_readout=16, max_ctx=8300,
                      pages=1024)
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    long_prompt = synth.prompt_tokens(1, 500, long_len, shape.vocab)
    shorts = [synth.prompt_tokens(1, 501 + s, short_len, shape.vocab) for s in range(n_short)]
    say("long decode: oracle")
    sess_long = Session(w, num)
    sess_long.step(long_prompt, readout=[])
    sess_short = []
    for s in range(n_short):
        ss = Session(w, num)
        ss.step(shorts[s], readout=[])
        sess_short.append(ss)
    feed = synth.prompt_tokens(1, 520, 3, shape.vocab)
    ref_alone = sess_long.step([int(feed[0])])[0]
    ref_batch = [sess_long.step([int(feed[1])])[0]] + [sess_short[s].step([int(feed[2])])[0] for s in range(n_short)]
    say("long decode: gpu")
    wl = rt.alloc()
    rt.forward([Pass(wl, long_prompt)])
    ws = [rt.alloc() for _ in range(n_short)]
    rt.forward([Pass(ws[s], shorts[s]) for s in range(n_short)])
    rep = Report()
    toks, lg = rt.forward([Pass(wl, [int(feed[0])], [0], [(0, 1.0, 0)])], want_logits=True)
    t, m = apply(ref_alone, 0)
    rep.add(toks[0], t, m, tau_for(0, 1.0), lg[0], ref_alone, ("alone",))
    toks, lg = rt.forward([Pass(wl, [int(feed[1])], [0], [(0, 1.0, 0)])] +
                          [Pass(ws[s], [int(feed[2])], [0], [(0, 1.0, 0)]) for s in range(n_short)],
                          want_logits=True)
    for i in range(n_short + 1):
        t, m = apply(ref_batch[i], 0)
        rep.add(toks[i], t, m, tau_for(0, 1.0), lg[i], ref_batch[i], ("batch", i))
    rep.check()
    rt.close()


def test_no_launch_flag_is_refused_on_a_gpu_context(torch_cuda):
    """Planning without running would commit tokens whose KV was never
    computed: a context with weights refuses it and changes nothing."""
    from paged_kv_forward_amd import _native as N
    from paged_kv_forward_amd.runtime import Pass
    recipe = RECIPES["gains1"]
    rt = make_runtime(recipe.shape, recipe, torch_cuda)
    ws = rt.alloc()
    before = rt.pool_stats()
    with pytest.raises(N.PieError):
        rt.forward([Pass(ws, [1, 2, 3], [2], [(0, 1.0, 0)])], flags=N.PIE_FLAG_NO_LAUNCH)
    assert rt.ws_info(ws)["len"] == 0 and rt.pool_stats() == before
    rt.close()


MID = synth.ModelShape("mid-2l", n_layers=2, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, d_ffn=2048,
                       vocab=4096)


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("width", [1024, 4608])
def test_mid_decode_both_qkv_forms_and_split_attention(torch_cuda, kv, width):
    """2-layer models of width 1024 and 4608 at head dim 128.  At 1024 the
    decode-sized QKV projection is one launch (narrow tiles with RoPE and the
    K/V append in their epilogue); at 4608 (K above 4096) it runs split-K,
    its partials summed by the reduce kernel, which applies RoPE and appends
    K/V.  Three sequences (40, 300 and 1100 tokens, the long one cut into
    several attention pieces merged by the combine kernel), three teacher-fed
    decode steps, bf16 or e4m3 KV, against the oracle.  Bounds from the
    oracle's float32 twin over the same rows (2e-2 where the twin stays below
    it): at width 4608 float32 accumulation alone moves these logits past
    2e-2."""
    import oracle.model as oracle_model
    from paged_kv_forward_amd.runtime import Pass
    shape = dataclasses.replace(MID, kv_dtype=kv, d_model=width, n_q_heads=width // 128,
                                n_kv_heads=2 if width == 1024 else 4)
    recipe = synth.WeightRecipe(shape, weight_seed=7, gain_std=0.02)
    lens = [40, 300, 1100]
    prompts = [synth.prompt_tokens(1, 600 + s, lens[s], shape.vocab) for s in range(3)]
    teach = [synth.prompt_tokens(1, 610 + s, 3, shape.vocab) for s in range(3)]
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)

    def oracle_rows():
        out = []
        for s in range(3):
            sess = Session(w, num)
            sess.step(prompts[s], readout=[])
            out.append([sess.step([int(teach[s][k])])[0] for k in range(3)])
        return out

    say("mid width %d kv=%d: oracle and its float32 twin" % (width, kv))
    ref = oracle_rows()
    plain = oracle_model.matmul_t
    oracle_model.matmul_t = lambda a, m: (np.asarray(a, np.float32) @ np.asarray(m, np.float32).T).astype(np.float64)
    try:
        twin = oracle_rows()
    finally:
        oracle_model.matmul_t = plain
    d = np.abs(np.array(ref) - np.array(twin))
    tol, tau, mean_tol = twin_bounds(float(d.max()), float(d.mean()))
    rt = make_runtime(shape, recipe, torch_cuda, max_rows=1500, max_seqs=4, max_readout=4, max_ctx=1200, pages=256)
    ws = [rt.alloc() for _ in range(3)]
    rt.forward([Pass(ws[s], prompts[s]) for s in range(3)])
    rep = Report()
    for k in range(3):
        toks, lg = rt.forward([Pass(ws[s], [int(teach[s][k])], [0], [(0, 1.0, 0)]) for s in range(3)],
                              want_logits=True)
        for s in range(3):
            t, m = apply(ref[s][k], 0)
            rep.add(toks[s], t, m, tau, lg[s], ref[s][k], ("mid", k, s))
    rep.check(tol=tol, mean_tol=mean_tol)
    rt.close()


def test_mid_prefill_fork_at_partial_page_and_chunked(torch_cuda):
    """Prefill at head dim 128 with masking away from the diagonal: a
    150-token prefix (its last page holds 6 tokens) forked twice, the
    children's suffixes (300 and 133 tokens) prefilled in one launch, so that
    their page tables hold a partly filled page in the middle; and a
    370-token prompt prefilled as 200 + 170 tokens, whose second chunk starts
    inside a page.  Readouts spread over each chunk (first token, both sides
    of a 64-token item boundary, the last token), against the oracle."""
    from paged_kv_forward_amd.runtime import Pass
    shape = MID
    recipe = synth.WeightRecipe(shape, weight_seed=9, gain_std=0.02)
    pre = synth.prompt_tokens(1, 700, 150, shape.vocab)
    sufs = [synth.prompt_tokens(1, 701, 300, shape.vocab), synth.prompt_tokens(1, 702, 133, shape.vocab)]
    longp = synth.prompt_tokens(1, 703, 370, shape.vocab)
    reads = [[0, 63, 64, 150, 299], [0, 5, 6, 70, 132]]
    rq = [0, 7, 8, 100, 169]
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    say("mid prefill fork/chunked: oracle")
    tree = [Chunk(pre, np.arange(150), -1, []),
            Chunk(sufs[0], 150 + np.arange(300), 0, reads[0]),
            Chunk(sufs[1], 150 + np.arange(133), 0, reads[1]),
            Chunk(longp[:200], np.arange(200), -1, []),
            Chunk(longp[200:], 200 + np.arange(170), 3, rq)]
    ref = forward_chunks(w, tree, num)
    rt = make_runtime(shape, recipe, torch_cuda, max_rows=1500, max_seqs=4, max_readout=16, max_ctx=1200, pages=256)
    p, q = rt.alloc(), rt.alloc()
    rt.forward([Pass(p, pre), Pass(q, longp[:200])])
    kids = [rt.fork(p) for _ in range(2)]
    passes = [Pass(kids[b], sufs[b], reads[b], [(0, 1.0, 0)] * len(reads[b])) for b in range(2)]
    passes.append(Pass(q, longp[200:], rq, [(0, 1.0, 0)] * len(rq)))
    toks, logits = rt.forward(passes, want_logits=True)
    assert rt.pool_stats()["kv_bytes_copied"] == 0
    rep = Report()
    row = 0
    for ci, rs in ((1, reads[0]), (2, reads[1]), (4, rq)):
        for k, r in enumerate(rs):
            t, m = apply(ref[ci][k], 0)
            rep.add(toks[row], t, m, tau_for(0, 1.0), logits[row], ref[ci][k], ("chunk", ci, r))
            row += 1
    rep.check()
    rt.close()


def test_tiny_prefill_past_the_page_id_table(torch_cuda):
    """A 33000-token prompt: 2063 pages, more than the 2048 page ids the bf16
    prefill attention keeps in LDS, so its last launch reads page ids with
    scalar loads.  Four launches of 8192 tokens, then the last 232 with three
    readouts, against stored oracle values (tests/golden/tiny_long_prefill.npz,
    written by tests/golden/make_golden.py tinylong)."""
    import os
    from paged_kv_forward_amd.runtime import Pass
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_long_prefill.npz")
    if not os.path.exists(path):
        pytest.skip("stored oracle values tiny_long_prefill not generated")
    g = np.load(path, allow_pickle=False)
    recipe = RECIPES["gains_spread"]
    shape = recipe.shape
    L, last0 = int(g["meta_prompt_len"]), int(g["meta_last_chunk"])
    toks = synth.prompt_tokens(1, int(g["meta_prompt_seed"]), L, shape.vocab)
    reads = [int(r) for r in g["row_step"]]
    rt = make_runtime(shape, recipe, torch_cuda, max_rows=8192, max_seqs=2, max_readout=4, max_ctx=L + 16,
                      pages=L // 16 + 8)
    ws = rt.alloc()
    for b in range(0, last0, 8192):
        rt.forward([Pass(ws, toks[b:b + 8192])])
    out, logits = rt.forward([Pass(ws, toks[last0:], reads, [(0, 1.0, 0)] * len(reads))], want_logits=True)
    rep = Report()
    for i, r in enumerate(reads):
        rep.add(out[i], int(g["token"][i]), float(g["margin"][i]), tau_for(0, 1.0), logits[i], g["logits_full"][i],
                ("long", r))
    rep.check()
    rt.close()
