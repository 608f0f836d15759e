"""Measures how strongly the full-depth random-init models amplify a tiny
change of their input, using the oracle alone.

Two implementations that both round to bf16 at the same storage points but
sum in different orders (fp32 on the GPU, fp64 in the oracle) round a few
values to neighbouring bf16 numbers; the question is how far such one-ulp
differences travel through 32 (or 80) layers.  This script runs the oracle
on one sequence of a workload twice: as is, and with one bf16 ulp added to a
seeded 0.1 % of the embedding values, and stores the largest and the mean
absolute change of the logits of the read-out rows.

    python tests/golden/conditioning.py c2 [c5]

Output: tests/golden/conditioning_<name>.json
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle.run import Chunk, SynthWeights, default_numerics, forward_chunks  # noqa: E402

FRACTION = 1e-3


def measure(config_id, name, decode_steps=3, seq=0):
    wl = synth.workload(config_id)
    shape = wl.shape
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    toks = np.concatenate([wl.prompt(seq), synth.teacher_tokens(config_id, seq, decode_steps, shape.vocab)])
    n = len(toks)
    chunk = Chunk(toks, np.arange(n), -1, list(range(wl.prompt_len[seq] - 1, n)))
    t0 = time.time()
    base = forward_chunks(w, [chunk], num)[0]
    embed = w.embed_rows
    rng = np.random.default_rng(synth.key_of("conditioning/%s" % name))

    def nudged(t):
        e = embed(t).astype(np.float32).copy()
        hit = rng.random(e.shape) < FRACTION
        e[hit] = e[hit] * np.float32(1.0 + 2.0 ** -7)  # one bf16 ulp (exact in bf16)
        return e

    w.embed_rows = nudged
    moved = forward_chunks(w, [chunk], num)[0]
    d = np.abs(base - moved)
    out = {"config": name, "model": shape.name, "n_layers": shape.n_layers, "seq": seq,
           "context": int(wl.prompt_len[seq]), "rows": int(base.shape[0]),
           "nudged_fraction_of_embedding_values": FRACTION, "nudge": "one bf16 ulp",
           "logit_std": float(base.std()), "max_abs_dlogit": float(d.max()),
           "mean_abs_dlogit": float(d.mean()), "oracle_seconds": round(time.time() - t0, 1)}
    path = os.path.join(HERE, "conditioning_%s.json" % name)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    for arg in sys.argv[1:] or ["c2"]:
        measure(int(arg[1:]), arg)
