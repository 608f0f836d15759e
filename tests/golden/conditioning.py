"""Measures the noise floor of float32 accumulation for each model and depth,
using the oracle alone.

The oracle computes in float64 and rounds to bf16 (or e4m3) at the storage
points the GPU uses.  An implementation that follows the same definition and
the same storage points but sums in float32, in another order, rounds a few
values to the neighbouring bf16 number, and these random-init models carry
such one-ulp differences far: at the 8B width even 2 layers move the logits
by more than 2e-2.  This script runs the oracle twice on one sequence of a
workload -- as is, and with its weight products (every q/k/v/o, gate/up/down
and lm_head matmul) taken in float32 by BLAS -- and stores the largest and the
mean absolute difference of the logits of the read-out rows.  The parity
bounds of the full-size tests are set from these numbers (tests/parity.py).

    python tests/golden/conditioning.py c2:2 c5:2 c3:2 c2 c5@512

"cN:L" cuts the model to its first L layers; "@C" shortens the prompt to C
tokens (to keep the 80-layer run affordable).  Output:
tests/golden/conditioning_<name>.json
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
import oracle.model as oracle_model  # noqa: E402
from oracle.run import Chunk, SynthWeights, default_numerics, forward_chunks  # noqa: E402


def matmul_f32(a, w):
    """The oracle's weight product with float32 inputs and float32 accumulation."""
    return (np.asarray(a, dtype=np.float32) @ np.asarray(w, dtype=np.float32).T).astype(np.float64)


def measure(arg, decode_steps=3):
    spec, _, ctx = arg.partition("@")
    cfg, _, layers = spec.partition(":")
    config_id = int(cfg[1:])
    wl = synth.workload(config_id)
    shape = wl.shape if not layers else synth.first_layers(wl.shape, int(layers))
    if config_id == 3:  # one branch: the shared prefix, then its suffix
        toks = np.concatenate([wl.prefix(), wl.prompt(0)])
        n_prompt = len(toks)
    else:
        toks = wl.prompt(0)
        n_prompt = len(toks)
    if ctx:
        toks, n_prompt = toks[:int(ctx)], int(ctx)
    toks = np.concatenate([toks, synth.teacher_tokens(config_id, 0, decode_steps, shape.vocab)])
    n = len(toks)
    chunk = Chunk(toks, np.arange(n), -1, list(range(n_prompt - 1, n)))
    w = SynthWeights(synth.WeightRecipe(shape))
    num = default_numerics(shape)
    t0 = time.time()
    base = forward_chunks(w, [chunk], num)[0]
    plain = oracle_model.matmul_t
    oracle_model.matmul_t = matmul_f32
    try:
        twin = forward_chunks(w, [chunk], num)[0]
    finally:
        oracle_model.matmul_t = plain
    d = np.abs(base - twin)
    name = "c%d%s%s" % (config_id, "_first%s" % layers if layers else "", "_ctx%s" % ctx if ctx else "")
    out = {"name": name, "model": shape.name, "n_layers": shape.n_layers, "context": n_prompt,
           "rows": int(base.shape[0]), "logit_std": float(base.std()),
           "twin": "weight products in float32", "max_abs_dlogit": float(d.max()),
           "mean_abs_dlogit": float(d.mean()), "oracle_seconds": round(time.time() - t0, 1)}
    with open(os.path.join(HERE, "conditioning_%s.json" % name), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    for a in sys.argv[1:] or ["c2:2"]:
        measure(a)
