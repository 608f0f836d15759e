"""Writes the stored expected values of the full-size GPU parity tests.

Calls only the oracle (oracle/) and the seeded input generator (synth/).  Every
decode step of a checked sequence is fed a seeded "teacher" token, so the
whole trajectory of a sequence is one chunk of known tokens and the oracle can
run it layer-major in one pass (weights drawn once per layer); the GPU test
feeds the same tokens.  By the incremental-decode invariant of the oracle,
reading out row i of that chunk equals decoding token by token.

    python tests/golden/make_golden.py c2 [c3 c4 c4long c5 c5ctx512 tinylong] [c2:1 ...]

"cN:L" writes the same case for the model cut to its first L layers
(<name>_first<L>.npz).  The checked rows follow the sampling plan of the
parity tests: the 8B decode checks sequences 0, 21, 42 and 63 at every one of
their 129 readouts; the fork checks the prefix's own readout and branches 0,
4 and 9 over the suffix and all 64 Gumbel steps; the mix checks prompts 0 and
7 and the shortest, a middle and the longest decode row; the 70B decode
checks one sequence at the full 4096-token context and, with the prompt cut
to 512 tokens, four sequences over 96 steps each (enough rows for some
oracle margins to clear the 80-layer noise floor).

Output: tests/golden/<name>.npz with, per checked readout row, the oracle's
token, its top-2 margin, the float32 logits at a fixed seeded subset of
vocabulary indices, and the full float32 logits for a few rows.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle.epilogue import scores, top2_margin, argmax_lowest  # noqa: E402
from oracle.run import Chunk, SynthWeights, default_numerics, forward_chunks  # noqa: E402

SUBSET = 2048  # logits kept for every row at these seeded vocabulary indices


def subset_idx(vocab):
    return np.sort(synth.uniform_int(SUBSET, synth.key_of("golden/subset"), 0, vocab))


teacher_tokens = synth.teacher_tokens


LAYERS = None  # set by "cN:L" on the command line


def matmul_f32(a, w):
    """The oracle's weight product with float32 inputs and float32 accumulation
    (the float32 twin of tests/golden/conditioning.py)."""
    return (np.asarray(a, dtype=np.float32) @ np.asarray(w, dtype=np.float32).T).astype(np.float64)


def run(w, chunks, num):
    """The oracle's logits for the chunks and, for the cut models (cheap), the
    same run with every weight product in float32: the twin's difference over
    exactly the stored rows bounds the GPU's (tests/parity.py)."""
    logits = forward_chunks(w, chunks, num)
    if LAYERS is None:
        return logits, None
    import oracle.model as om
    plain = om.matmul_t
    om.matmul_t = matmul_f32
    try:
        twin = forward_chunks(w, chunks, num)
    finally:
        om.matmul_t = plain
    return logits, twin


def model(wl):
    """The workload's model, cut to LAYERS layers when asked."""
    return wl.shape if LAYERS is None else synth.first_layers(wl.shape, LAYERS)


def finish(name, rows, full_rows, vocab, meta):
    """rows: list of dicts (seq, step, kind, temp, seed, lane, logits[, twin])."""
    if LAYERS is not None:
        name = "%s_first%d" % (name, LAYERS)
        meta = dict(meta, n_layers=LAYERS)
    idx = subset_idx(vocab)
    out = {"subset_idx": idx}
    toks, margins, subs = [], [], []
    for r in rows:
        s32, s64 = scores(r["logits"], r["kind"], r["temp"], r["seed"], r["lane"])
        toks.append(argmax_lowest(s32))
        margins.append(top2_margin(s64))
        subs.append(r["logits"][idx].astype(np.float32))
    out["token"] = np.array(toks, dtype=np.int32)
    out["margin"] = np.array(margins)
    out["logits_subset"] = np.stack(subs)
    out["row_seq"] = np.array([r["seq"] for r in rows], dtype=np.int32)
    out["row_step"] = np.array([r["step"] for r in rows], dtype=np.int32)
    out["row_kind"] = np.array([r["kind"] for r in rows], dtype=np.int32)
    out["full_rows"] = np.array(full_rows, dtype=np.int32)
    out["logits_full"] = np.stack([rows[i]["logits"].astype(np.float32) for i in full_rows])
    if rows and rows[0].get("twin") is not None:
        d = np.concatenate([np.abs(r["logits"] - r["twin"]) for r in rows])
        out["twin_max_abs_dlogit"] = np.asarray(float(d.max()))
        out["twin_mean_abs_dlogit"] = np.asarray(float(d.mean()))
        print("%s: float32 twin over the stored rows: max %.4g mean %.4g" % (name, d.max(), d.mean()))
    for k, v in meta.items():
        out["meta_" + k] = np.asarray(v)
    path = os.path.join(HERE, name + ".npz")
    np.savez_compressed(path, **out)
    print("wrote", path, "rows", len(rows), "excluded(margin<2e-2)",
          int(np.sum(out["margin"] < 2e-2)), flush=True)


def c2(decode_steps=None, seqs=(0, 21, 42, 63)):
    """Llama-3.1-8B decode: sequences of 2048 prompt tokens + teacher-fed decode steps
    (all 128 at full depth; 3 when cut to 2 layers, 8 when cut to 1)."""
    wl = synth.workload(2)
    shape = model(wl)
    if decode_steps is None:
        decode_steps = {None: wl.decode_steps, 2: 3, 1: 8}.get(LAYERS, 8)
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    chunks = []
    for s in seqs:
        toks = np.concatenate([wl.prompt(s), teacher_tokens(2, s, decode_steps, shape.vocab)])
        n = len(toks)
        ro = list(range(wl.prompt_len[s] - 1, n))
        chunks.append(Chunk(toks, np.arange(n), -1, ro))
    t0 = time.time()
    logits, twin = run(w, chunks, num)
    print("c2 oracle %.0f s" % (time.time() - t0), flush=True)
    rows = []
    for ci, s in enumerate(seqs):
        for k in range(decode_steps + 1):
            rows.append(dict(seq=s, step=k, kind=synth.EPI_ARGMAX, temp=1.0, seed=0, lane=0,
                             logits=logits[ci][k], twin=None if twin is None else twin[ci][k]))
    per = decode_steps + 1
    full = sorted({0, decode_steps, per, 2 * per - 1, len(rows) - 1})
    finish("c2_decode_8b", rows, full, shape.vocab,
           dict(seqs=list(seqs), decode_steps=decode_steps))


def c3(decode_steps=None, branches=(0, 4, 9)):
    """Fork at the 8B shape: 8192-token prefix (read out at its last token with
    argmax), 256-token suffix per branch, Gumbel-max at T=0.7 over the suffix's
    readout and every decode step (64 at full depth; 2 when cut to 2 layers)."""
    wl = synth.workload(3)
    shape = model(wl)
    if decode_steps is None:
        decode_steps = 2 if LAYERS == 2 else wl.decode_steps
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    pre = wl.prefix()
    P = len(pre)
    with_prefix = LAYERS != 2
    chunks = [Chunk(pre, np.arange(P), -1, [P - 1] if with_prefix else [])]
    for b in branches:
        toks = np.concatenate([wl.prompt(b), teacher_tokens(3, b, decode_steps, shape.vocab)])
        n = len(toks)
        chunks.append(Chunk(toks, P + np.arange(n), 0, list(range(wl.prompt_len[b] - 1, n))))
    t0 = time.time()
    logits, twin = run(w, chunks, num)
    print("c3 oracle %.0f s" % (time.time() - t0), flush=True)
    rows = []
    if with_prefix:
        # the prefix pass's own readout: sequence -1, step -1, argmax
        rows.append(dict(seq=-1, step=-1, kind=synth.EPI_ARGMAX, temp=1.0, seed=0, lane=0,
                         logits=logits[0][0], twin=None if twin is None else twin[0][0]))
    for ci, b in enumerate(branches):
        for k in range(decode_steps + 1):
            rows.append(dict(seq=b, step=k, kind=synth.EPI_GUMBEL, temp=0.7,
                             seed=synth.epilogue_seed(wl.branch_seed[b], k), lane=0,
                             logits=logits[1 + ci][k], twin=None if twin is None else twin[1 + ci][k]))
    full = sorted({0, 1, decode_steps + 1, len(rows) - 1})
    finish("c3_fork_8b", rows, full, shape.vocab,
           dict(branches=list(branches), decode_steps=decode_steps, prefix_readout=int(with_prefix)))


def c4(seqs=None, name="c4_mix_8b"):
    """Mix at the 8B shape: prompts 0 and 7 (4096 tokens, read out at the end of the
    last 512-chunk), and decode rows (the shortest context, one other and -- cut to
    1 layer -- the longest) read out at each of the 8 launches."""
    wl = synth.workload(4)
    shape = model(wl)
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    dec_ctx = np.array(wl.prompt_len[8:])
    shortest = 8 + int(np.argmin(dec_ctx))
    longest = 8 + int(np.argmax(dec_ctx))
    other = 8 + 37
    if seqs is None:
        seqs = [0, 7, shortest, other] + ([longest] if LAYERS == 1 else [])
    chunks, meta_rows = [], []
    for s in seqs:
        if s < 8:
            toks = wl.prompt(s)
            chunks.append(Chunk(toks, np.arange(len(toks)), -1, [len(toks) - 1]))
            meta_rows.append([(s, 7)])
        else:
            ctx = wl.prompt(s)
            toks = np.concatenate([ctx, teacher_tokens(4, s, 8, shape.vocab)])
            n = len(toks)
            # the context is prefilled in setup; launch k feeds teacher token k
            chunks.append(Chunk(toks, np.arange(n), -1, list(range(len(ctx), n))))
            meta_rows.append([(s, k) for k in range(8)])
    t0 = time.time()
    logits, twin = run(w, chunks, num)
    print("c4 oracle %.0f s" % (time.time() - t0), flush=True)
    rows = []
    for ci, s in enumerate(seqs):
        for j, (_, k) in enumerate(meta_rows[ci]):
            rows.append(dict(seq=s, step=k, kind=wl.epi_kind[s], temp=1.0,
                             seed=synth.epilogue_seed(wl.branch_seed[s], k), lane=0,
                             logits=logits[ci][j], twin=None if twin is None else twin[ci][j]))
    finish(name, rows, sorted({0, 1, 2, len(rows) - 1}), shape.vocab, dict(seqs=seqs))


def c4long():
    """The mix's longest-context decode row (context 8147), stored apart from the
    other checked rows of the full-depth mix (c4_mix_8b_long.npz)."""
    wl = synth.workload(4)
    longest = 8 + int(np.argmax(np.array(wl.prompt_len[8:])))
    c4(seqs=[longest], name="c4_mix_8b_long")


def c5(decode_steps=None, seqs=None, ctx=None, name="c5_decode_70b"):
    """Llama-3.3-70B decode with e4m3 KV: the prompt (4096 tokens, or its first
    `ctx`) + teacher-fed decode steps."""
    wl = synth.workload(5)
    shape = model(wl)
    if decode_steps is None:
        decode_steps = 8 if LAYERS == 1 else 2
    if seqs is None:
        seqs = (0, 31) if LAYERS == 1 else (0,)
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    n_prompt = ctx or wl.prompt_len[0]
    chunks = []
    for s in seqs:
        toks = np.concatenate([wl.prompt(s)[:n_prompt], teacher_tokens(5, s, decode_steps, shape.vocab)])
        n = len(toks)
        chunks.append(Chunk(toks, np.arange(n), -1, list(range(n_prompt - 1, n))))
    t0 = time.time()
    logits, twin = run(w, chunks, num)
    print("c5 oracle %.0f s" % (time.time() - t0), flush=True)
    rows = []
    for ci, s in enumerate(seqs):
        for k in range(decode_steps + 1):
            rows.append(dict(seq=s, step=k, kind=synth.EPI_ARGMAX, temp=1.0, seed=0, lane=0,
                             logits=logits[ci][k], twin=None if twin is None else twin[ci][k]))
    meta = dict(seqs=list(seqs), decode_steps=decode_steps)
    if ctx:
        meta["ctx"] = ctx
    finish(name, rows, sorted({0, decode_steps, len(rows) - 1}), shape.vocab, meta)


def c5ctx512():
    """The 70B decode with every prompt cut to its first 512 tokens: four
    sequences, 96 decode steps each (388 readouts)."""
    c5(decode_steps=96, seqs=(0, 10, 21, 31), ctx=512, name="c5_decode_70b_ctx512")


def tinylong():
    """The tiny model prefilling one 33000-token prompt (more pages than the
    prefill attention kernel keeps in LDS, 2063 against 2048): read out at 3
    rows of its last 232 tokens, which the GPU test prefills as the fifth
    launch after four of 8192 tokens.  The oracle runs it in 2048-token
    chunks (same KV, by its chunk-boundary invariant)."""
    recipe = synth.WeightRecipe(synth.TINY, weight_seed=99, gain_std=0.02)
    shape = recipe.shape
    L, last0, reads = 33000, 4 * 8192, [0, 100, 231]
    toks = synth.prompt_tokens(1, 800, L, shape.vocab)
    w = SynthWeights(recipe, cache_layers=True)
    num = default_numerics(shape)
    tree, b = [], 0
    while b < last0:
        e = min(b + 2048, last0)
        tree.append(Chunk(toks[b:e], np.arange(b, e), len(tree) - 1, []))
        b = e
    tree.append(Chunk(toks[last0:], np.arange(last0, L), len(tree) - 1, reads))
    t0 = time.time()
    out = forward_chunks(w, tree, num)[-1]
    print("tinylong oracle %.0f s" % (time.time() - t0), flush=True)
    rows = [dict(seq=0, step=r, kind=0, temp=1.0, seed=0, lane=i, logits=out[i]) for i, r in enumerate(reads)]
    finish("tiny_long_prefill", rows, [0, 1, 2], shape.vocab,
           {"prompt_len": L, "last_chunk": last0, "prompt_seed": 800})


if __name__ == "__main__":
    for arg in sys.argv[1:] or ["c2"]:
        name, _, layers = arg.partition(":")
        LAYERS = int(layers) if layers else None
        globals()[name]()
