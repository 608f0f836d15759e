"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, against stored oracle values (tests/golden/*.npz, written by
tests/golden/make_golden.py from the oracle alone).

Checked sequences are fed seeded teacher tokens at every decode step (the
others are computed in the same launches but not compared).
"""
import os

import numpy as np
import pytest

import synth
from tests.parity import Report, say, tau_for

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip("stored oracle values %s not generated" % name)
    return np.load(path, allow_pickle=False)


def compare(rep, g, row, tok, logits, tag):
    kind = int(g["row_kind"][row])
    tau = tau_for(kind, 0.7 if kind else 1.0)
    sub = logits[g["subset_idx"]]
    err = float(np.max(np.abs(sub - g["logits_subset"][row])))
    rep.max_err = max(rep.max_err, err)
    fr = list(g["full_rows"])
    if row in fr:
        full = g["logits_full"][fr.index(row)]
        rep.max_err = max(rep.max_err, float(np.max(np.abs(logits - full))))
    rep.add(tok, g["token"][row], float(g["margin"][row]), tau, tag=tag)


def test_c2_llama8b_decode_batch64():
    import torch
    from paged_kv_forward_amd.runtime import Pass, PieRuntime, upload_weights
    g = golden("c2_decode_8b")
    wl = synth.workload(2)
    shape = wl.shape
    steps = int(g["meta_decode_steps"])
    checked = list(g["meta_seqs"])
    say("c2: uploading 8B weights")
    w = upload_weights(synth.WeightRecipe(shape))
    n = wl.n_seqs
    max_ctx = wl.prompt_len[0] + steps + 8
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * 2
    pages = n * ((max_ctx + 15) // 16 + 1)
    rt = PieRuntime(shape, w, pages * page_bytes, max_rows=4 * 2048, max_seqs=n, max_readout=n,
                    max_ctx=max_ctx)
    ws = [rt.alloc() for _ in range(n)]
    rep = Report()
    logits_dev = torch.empty((n, shape.vocab), dtype=torch.float32, device="cuda")
    say("c2: prefill 64 x 2048 in launches of 4 sequences")
    for b in range(0, n, 4):
        ss = list(range(b, b + 4))
        toks, _ = rt.forward([Pass(ws[s], wl.prompt(s), [wl.prompt_len[s] - 1], [(0, 1.0, 0)]) for s in ss],
                             logits_out=logits_dev[:4])
        lg = logits_dev[:4].cpu().numpy()
        for j, s in enumerate(ss):
            if s in checked:
                row = checked.index(s) * (steps + 1)
                compare(rep, g, row, toks[j], lg[j], ("prefill", s))
    teach = [synth.teacher_tokens(2, s, steps, shape.vocab) for s in range(n)]
    for k in range(steps):
        say("c2: decode step", k + 1)
        toks, _ = rt.forward([Pass(ws[s], [int(teach[s][k])], [0], [(0, 1.0, 0)]) for s in range(n)],
                             logits_out=logits_dev)
        lg = logits_dev.cpu().numpy()
        for ci, s in enumerate(checked):
            compare(rep, g, ci * (steps + 1) + k + 1, toks[s], lg[s], ("decode", k + 1, s))
    rep.check()
    rt.close()
