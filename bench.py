"""Decode benchmark of the batched paged-KV forward pass on one MI355X.

Workload (synthetic, seeded): the Llama-3.1-8B shape (32 layers, d 4096,
32 q / 8 kv heads, head_dim 128, ffn 14336, vocab 128256), bf16 weights
N(0, 0.02), bf16 paged KV (page 16).  64 sequences of 2048 uniform random
prompt tokens are prefilled (setup, reported as prefill tokens/s), then greedy
(argmax) decode steps run with batch 64, each sequence feeding back its own
token.  A step is one pie_forward over the 64 decode rows: host packing, the
whole forward, the fused argmax epilogue and the token copy-back.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints one JSON line.  The decode-attention kernel's achieved HBM bandwidth
is measured with HIP events on the library's stream over the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PREFILL_TIMED_LAUNCHES = 4
N_SEQ = 64
PROMPT = 2048
PREFILL_SEQS_PER_LAUNCH = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, recipe, decode_rows=1, decode_steps=2, ctx=64, prefill_tokens=256, prefill_layers=2):
    """The oracle timed on the host cores, on bounded samples of the workload.

    decode: its incremental path (oracle.run.Session: token-major, contiguous
    per-layer KV), every layer's weights resident in host memory; `decode_rows`
    sequences with a `ctx`-token context (not timed) each take `decode_steps`
    one-token steps through all layers and the head.
    prefill: its layer-major pass (oracle.run.forward_chunks) over one
    `prefill_tokens`-token prompt through the first `prefill_layers` layers,
    scaled to all layers (the head is one readout row, timed apart)."""
    import synth
    from oracle.model import head_logits
    from oracle.run import Chunk, Session, SynthWeights, default_numerics, forward_chunks
    num = default_numerics(shape)
    w = SynthWeights(recipe, cache_layers=True)
    t0 = time.perf_counter()
    for l in range(shape.n_layers):
        w.layer(l)
    head, fin = w.head(), w.final_norm()
    t_draw = time.perf_counter() - t0
    # decode, incremental
    sess = []
    for r in range(decode_rows):
        s = Session(w, num)
        s.step(synth.prompt_tokens(2, 900 + r, ctx, shape.vocab), readout=[])
        sess.append(s)
    feed = synth.prompt_tokens(2, 950, decode_rows * decode_steps, shape.vocab)
    t0 = time.perf_counter()
    for k in range(decode_steps):
        for r, s in enumerate(sess):
            s.step([int(feed[k * decode_rows + r])])
    t_dec = time.perf_counter() - t0
    del sess
    # prefill, layer-major, over the first layers of the same resident weights
    cut = synth.first_layers(shape, prefill_layers)
    wc = SynthWeights(synth.WeightRecipe(cut, weight_seed=recipe.weight_seed, std=recipe.std,
                                         gain_std=recipe.gain_std))
    wc._layers = {l: w.layer(l) for l in range(prefill_layers)}
    wc._cache_layers = True
    wc._head, wc._final = head, fin
    toks = synth.prompt_tokens(2, 990, prefill_tokens, shape.vocab)
    t0 = time.perf_counter()
    h = forward_chunks(wc, [Chunk(toks, np.arange(prefill_tokens), -1, [])], num, want_hidden=True)[1][0]
    t_pre = time.perf_counter() - t0
    t0 = time.perf_counter()
    head_logits(h[-1:], fin, head, shape, num)
    t_head = time.perf_counter() - t0
    prefill_s = t_pre * shape.n_layers / prefill_layers + t_head
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    threads = min(threads, len(os.sched_getaffinity(0)))
    return {"value": round(decode_rows * decode_steps / t_dec, 4), "unit": "decode tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "decode: %d sequence(s) x %d one-token steps through all %d layers and the head on the "
                      "oracle's incremental path (float64 numpy, context %d tokens, weights resident), %.1f s; "
                      "prefill: one %d-token prompt through %d of %d layers on its layer-major pass, scaled "
                      "to all layers, %.1f s (weights drawn beforehand in %.1f s, not timed)" %
                      (decode_rows, decode_steps, shape.n_layers, ctx, t_dec, prefill_tokens, prefill_layers,
                       shape.n_layers, t_pre + t_head, t_draw),
            "prefill_value": round(prefill_tokens / prefill_s, 2), "prefill_unit": "prefill tokens/s"}


# ---------------------------------------------------------------- profiles
ATTN_SOURCES = ["paged_kv_forward_amd/csrc/attention.hip", "paged_kv_forward_amd/csrc/attention.h",
                "paged_kv_forward_amd/csrc/common.h"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "attn_decode_hbm_counters.json")
# back-to-back runs of each decode-attention launch in the roofline's timed pass
ATTN_REPS = 8
TRACE_CMD = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_c2 -o c2 -- "
             "python3 <repo>/bench.py --steps 20 --warmup 5 --no-cpu-baseline")
PMC_CMDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch -o f -- python3 <repo>/bench.py "
    "--steps 3 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_write -o w -- python3 <repo>/bench.py "
    "--steps 3 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_copy_f -o cf -- python3 <repo>/bench.py "
    "--calibrate-copy",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_copy_w -o cw -- python3 <repo>/bench.py "
    "--calibrate-copy"]


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name):
    return name.split("(")[0].replace("void ", "").strip()


def summarize_prefill(trace, prof):
    """Per-projection durations of the prefill GEMMs (8192 rows per launch)
    and of prefill attention, from the same kernel trace."""
    from synth import workload
    shape = workload(2).shape
    T = PREFILL_SEQS_PER_LAUNCH * PROMPT
    d, f_, hq, hk = shape.d_model, shape.d_ffn, shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    nk = {"qkv": (hq + 2 * hk, d), "o": (d, hq), "gate_up": (2 * f_, d), "down": (d, f_)}
    dur = {k: [] for k in nk}
    attn = []
    prev = None
    for r in trace:
        k = short_name(r["Kernel_Name"])
        if "embed_kernel" in k and int(r["Grid_Size_X"]) == N_SEQ * 256:
            break  # decode starts
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if k.startswith("pie::gemm_dma_kernel") or k.startswith("pie::gemm_big_kernel"):
            epi = k.split("<")[1].rstrip(">")
            proj = {"0": "qkv", "2": "gate_up"}.get(epi)
            if epi == "1":
                proj = "down" if prev == "gate_up" else "o"
            dur[proj].append(us)
            prev = proj
        elif k.startswith("pie::attn_prefill"):  # attn_prefill_h_kernel (bf16 KV) or attn_prefill_kernel (e4m3)
            attn.append(us)
            prev = "attn"
    rows = ["# Prefill kernels of the benchmark run (Llama-3.1-8B shape, 8192 rows per launch)", "",
            "Same run as `decode_llama8b_b64_kernel_trace.md`:", "", "    " + TRACE_CMD, "",
            "The prefill is 16 launches of 4 sequences x 2048 tokens (T = 8192 rows).  Each projection",
            "GEMM runs once per layer; flops = 2 T N K.  Peak: %.0f TFLOP/s (dense bf16 MFMA)." % PEAK_BF16_TFLOPS, "",
            "| kernel | projection (N x K) | launches | avg us | TFLOP/s | fraction of peak |",
            "|---|---|---|---|---|---|"]
    tot_f, tot_t = 0.0, 0.0
    for proj, (n, k) in nk.items():
        if not dur[proj]:
            continue
        avg = sum(dur[proj]) / len(dur[proj])
        tf = 2.0 * T * n * k / (avg * 1e-6) / 1e12
        tot_f += 2.0 * T * n * k * len(dur[proj])
        tot_t += sum(dur[proj]) * 1e-6
        kern = "gemm_dma_kernel<%s>" % {"qkv": 0, "o": 1, "gate_up": 2, "down": 1}[proj]
        rows.append("| `%s` | %s (%d x %d) | %d | %.1f | %.0f | %.3f |"
                    % (kern, proj, n, k, len(dur[proj]), avg, tf, tf / PEAK_BF16_TFLOPS))
    if tot_t:
        rows.append("| all four | | | | %.0f | %.3f |" % (tot_f / tot_t / 1e12, tot_f / tot_t / 1e12 / PEAK_BF16_TFLOPS))
    if attn:
        avg = sum(attn) / len(attn)
        fl = 4.0 * shape.n_q_heads * shape.head_dim * (PROMPT * (PROMPT + 1) / 2) * PREFILL_SEQS_PER_LAUNCH
        rows += ["", "Prefill attention (causal, 4 sequences of 2048 per launch): %d launches, avg %.1f us, "
                 "%.0f TFLOP/s." % (len(attn), avg, fl / (avg * 1e-6) / 1e12)]
    with open(os.path.join(prof, "prefill_llama8b_t8192_kernel_trace.md"), "w") as f:
        f.write("\n".join(rows) + "\n")


def summarize(out_dir):
    """Write the committed summaries under profiles/ from a rocprofv3 kernel
    trace (out_dir/trace_c2) and the FETCH_SIZE / WRITE_SIZE counter runs
    (out_dir/pmc_*) of this benchmark."""
    import csv
    import glob
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    stats = list(csv.DictReader(open(glob.glob(os.path.join(out_dir, "trace_c2", "*kernel_stats.csv"))[0])))
    lines = ["# Kernel trace of the decode benchmark (Llama-3.1-8B shape, batch 64)", "",
             "Command (on one MI355X, from the repository root):", "", "    " + TRACE_CMD, "",
             "The run includes the 64 x 2048-token prefill (16 launches of 4 sequences) and 68 decode",
             "steps (5 warm-up + 20 timed + 20 host-loop + 20 with HIP events, each decode-attention launch",
             "run %d times back to back there, + 3 per-class), then the" % ATTN_REPS,
             "FP8-weight variant (its own prefill and 28 decode steps; kernels `<..., true>`).  Per kernel:",
             "calls, average and total duration from `c2_kernel_stats.csv`.", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats[:24]:
        lines.append("| `%s` | %s | %.2f | %.2f | %.3f |" % (short_name(r["Name"]), r["Calls"],
                     float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    # one decode step from the trace: the launches from a 64-row embedding to the next
    trace = sorted(csv.DictReader(open(glob.glob(os.path.join(out_dir, "trace_c2", "*kernel_trace.csv"))[0])),
                   key=lambda r: int(r["Start_Timestamp"]))
    steps, cur = [], None
    for r in trace:
        if "embed_kernel" in r["Kernel_Name"]:
            cur = [] if int(r["Grid_Size_X"]) == N_SEQ * 256 else None
            if cur is not None:
                steps.append(cur)
        if cur is not None:
            cur.append(r)
    # decode steps with bf16 weights, then those of the FP8-weight variant
    # (their skinny GEMM launches are the FP8 instantiations)
    is_f8 = lambda st: any("gemm_skinny_kernel" in r["Kernel_Name"] and "true" in r["Kernel_Name"] for r in st)
    for label, group in (("bf16 weights", [st for st in steps if not is_f8(st)]),
                         ("FP8 projection and lm_head weights", [st for st in steps if is_f8(st)])):
        if len(group) < 3:
            continue
        st = group[len(group) // 2]
        span = (int(st[-1]["End_Timestamp"]) - int(st[0]["Start_Timestamp"])) / 1e3
        agg = {}
        for r in st:
            k = short_name(r["Kernel_Name"])
            a = agg.setdefault(k, [0, 0.0])
            a[0] += 1
            a[1] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        busy = sum(v[1] for v in agg.values())
        lines += ["", "One decode step with %s (the middle one of those in the run): %d launches, %.1f us from "
                  "the first kernel's start to the last one's end, %.1f us of it inside kernels."
                  % (label, len(st), span, busy),
                  "", "| kernel | launches per step | us per step |", "|---|---|---|"]
        for k, (n, d) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            lines.append("| `%s` | %d | %.1f |" % (k, n, d))
    # the roofline's timed pass of the traced run: bf16 decode steps 46-65
    # (5 warm-up, 20 timed, 20 host-loop steps before it)
    bf = [st for st in steps if not is_f8(st)]
    att = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for st in bf[45:65] for r in st if "attn_decode_kernel" in r["Kernel_Name"]]
    if att:
        lines += ["", "Decode attention in the pass that `bench.py` times its roofline over (bf16 decode steps "
                  "46-65 of this run): %d launches, average %.2f us in this trace." % (len(att), sum(att) / len(att))]
        # the traced run's own JSON line, when its output was kept as out_dir/trace.log
        log_path = os.path.join(out_dir, "trace.log")
        js = [l for l in open(log_path).read().splitlines() if l.startswith('{"metric"')] \
            if os.path.exists(log_path) else []
        if js:
            rf = json.loads(js[-1])["roofline"]
            lines.append("The same run's JSON line: `avg_launch_ms` %.5f (%.2f us), %s."
                         % (rf["avg_launch_ms"], rf["avg_launch_ms"] * 1e3, rf["timed_over"]))
    with open(os.path.join(prof, "decode_llama8b_b64_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    summarize_prefill(trace, prof)

    def per_kernel(csv_path):
        agg = {}
        for r in csv.DictReader(open(csv_path)):
            k = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            agg.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch = per_kernel(glob.glob(os.path.join(out_dir, "pmc_fetch", "*counter_collection.csv"))[0])
    write = per_kernel(glob.glob(os.path.join(out_dir, "pmc_write", "*counter_collection.csv"))[0])
    cf = per_kernel(glob.glob(os.path.join(out_dir, "pmc_copy_f", "*counter_collection.csv"))[0])
    cw = per_kernel(glob.glob(os.path.join(out_dir, "pmc_copy_w", "*counter_collection.csv"))[0])
    copy_kib = (1 << 30) / 1024.0
    cf_k = [v for k, v in cf.items() if "copyBuffer" in k[0]][0]
    cw_k = [v for k, v in cw.items() if "copyBuffer" in k[0]][0]
    f_scale, w_scale = copy_kib / cf_k, copy_kib / cw_k
    rows = ["# HBM bytes per dispatch of the decode kernels (Llama-3.1-8B shape, batch 64)", "",
            "Commands (on one MI355X, each its own run, from /tmp):", ""]
    rows += ["    " + c for c in PMC_CMDS]
    rows += ["", "Scale factors from the plain 1 GiB device copy (`bench.py --calibrate-copy`): "
             "FETCH_SIZE read %.1f KiB for 1048576 KiB moved (x %.4f), WRITE_SIZE %.1f KiB (x %.4f)."
             % (cf_k, f_scale, cw_k, w_scale), "",
             "Decode step contexts in these runs: 2049..2055 tokens.", "",
             "| kernel | grid (threads) | fetch KiB | write KiB | HBM MB per dispatch (scaled) |",
             "|---|---|---|---|---|"]
    attn = None
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if k[1] < 8192:
            continue
        fb, wb = fetch[k], write.get(k, 0.0)
        mb = (fb * f_scale + wb * w_scale) * 1024 / 1e6
        rows.append("| `%s` | %d | %.1f | %.1f | %.1f |" % (k[0], k[1], fb, wb, mb))
        if k[0].startswith("pie::attn_decode_kernel") and k[1] == 64 * 8 * 256:
            attn = {"kernel": k[0], "grid_threads": k[1], "fetch_kib": fb, "write_kib": wb,
                    "fetch_scale": f_scale, "write_scale": w_scale,
                    "bytes_per_dispatch": (fb * f_scale + wb * w_scale) * 1024,
                    "context_tokens": [2049, 2055]}
    with open(os.path.join(prof, "decode_llama8b_b64_hbm_counters.md"), "w") as f:
        f.write("\n".join(rows) + "\n")
    if attn:
        attn["sources_sha256"] = sources_digest(ATTN_SOURCES)
        with open(TRAFFIC_JSON, "w") as f:
            json.dump(attn, f, indent=1)
    print("wrote summaries under", prof)


def measured_traffic():
    """Counter-measured HBM bytes per decode-attention dispatch, or None when
    the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("sources_sha256") != sources_digest(ATTN_SOURCES):
        return None
    return t



def fp8_decode_summary(shape, K, W):
    """The FP8 variant measured beside the headline: the same decode workload
    (64 sequences of 2048 prompt tokens, argmax, loop-carried steps) with every
    layer projection block-scaled FP8 and decode streaming the FP8 copies."""
    import torch
    import synth
    from paged_kv_forward_amd import _native as N
    from paged_kv_forward_amd.runtime import Pass, PieRuntime, upload_weights
    recipe = synth.WeightRecipe(shape, fp8_blocks=True)
    wl = synth.workload(2)
    log("bench: FP8 variant: drawing and uploading weights")
    weights = upload_weights(recipe, "cuda:0", fp8=True)
    max_ctx = PROMPT + W + K + 3 + 8
    pages = N_SEQ * ((max_ctx + 15) // 16 + 1)
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * 2
    rt = PieRuntime(shape, weights, pages * page_bytes, max_rows=PREFILL_SEQS_PER_LAUNCH * PROMPT,
                    max_seqs=N_SEQ, max_readout=N_SEQ, max_ctx=max_ctx)
    ws = [rt.alloc() for _ in range(N_SEQ)]
    nxt = np.zeros(N_SEQ, dtype=np.int32)
    for b in range(0, N_SEQ, PREFILL_SEQS_PER_LAUNCH):
        ss = range(b, b + PREFILL_SEQS_PER_LAUNCH)
        toks, _ = rt.forward([Pass(ws[s], wl.prompt(s), [PROMPT - 1], [(0, 1.0, 0)]) for s in ss])
        nxt[b:b + PREFILL_SEQS_PER_LAUNCH] = toks
    ws_arr = np.array(ws, dtype=np.uint64)
    for _ in range(W):
        nxt[:] = rt.decode_step(ws_arr, nxt)
    ctx_first = rt.ws_info(ws[0])["len"] + 1
    tok_dev = torch.tensor(nxt, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        rt.decode_async(ws_arr, tok_dev, tok_dev)
    rt.sync()
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    nxt[:] = tok_dev.cpu().numpy()
    rt.profile_enable(N.KERNEL_CLASSES)
    for _ in range(3):
        nxt[:] = rt.decode_step(ws_arr, nxt)
    pb = rt.profile_read()
    rt.profile_enable([])
    rt.close()
    del weights
    torch.cuda.empty_cache()
    ms = t_dec / K * 1e3
    kv_tok = shape.n_kv_heads * shape.head_dim * 2 * 2
    proj = shape.n_layers * shape.d_model * (2 * shape.q_width + 2 * shape.kv_width + 3 * shape.d_ffn)
    fp8_params = proj + shape.vocab * shape.d_model  # projections and lm_head at one byte each
    wbytes = fp8_params + 4 * fp8_params // (128 * 128) + 2 * shape.d_model * (2 * shape.n_layers + 1)
    step_bytes = wbytes + sum(N_SEQ * (ctx_first + i) for i in range(K)) / K * kv_tok * shape.n_layers
    return {"value": round(N_SEQ * K / t_dec, 2), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "steps": K, "warmup": W,
            "weights": "layer projections and lm_head block-scaled FP8 (OCP e4m3 codes, one power-of-two "
                       "scale per 128x128 block) streamed by decode; embedding and norms bf16",
            "step_hbm": {"bytes_per_step": int(step_bytes),
                         "achieved_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1),
                         "frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
            "ms_per_step_by_kernel": {k: round(v[0] / 3, 4) for k, v in pb.items() if v[1]}}


def bench_70b(steps, warmup):
    """Decode at the Llama-3.3-70B shape (workload 5: 32 sequences of 4096
    prompt tokens, e4m3 KV with per-head scales, argmax, loop-carried steps),
    once with the bf16 weights and once with their block-scaled FP8 copies
    attached.  The FP8 copies are made on the device by pie_pack_weight_fp8,
    which rounds each weight to its block's nearest code (drawing an exactly
    FP8-representable 70B model on the host would take minutes), so the two
    runs time the same shapes on slightly different weights.  Prints one
    JSON line."""
    import torch
    import synth
    from paged_kv_forward_amd.runtime import Pass, PieRuntime, upload_weights
    torch.cuda.set_device(0)
    shape = synth.LLAMA_70B
    wl = synth.workload(5)
    recipe = synth.WeightRecipe(shape)
    t0 = time.perf_counter()
    log("bench 70b: drawing and uploading %.1f B weights with FP8 copies" % (shape.n_params() / 1e9))
    weights = upload_weights(recipe, "cuda:0", progress=lambda l: (l % 16 == 15) and log("  layer", l + 1),
                             fp8=True)
    log("bench 70b: weights ready in %.1f s" % (time.perf_counter() - t0))
    n, plen = wl.n_seqs, wl.prompt_len[0]
    K, W = steps, warmup
    max_ctx = plen + W + K + 8
    pages = n * ((max_ctx + 15) // 16 + 1)
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim  # e4m3: one byte
    per_launch = 2
    kv_tok = shape.n_kv_heads * shape.head_dim * 2 * shape.n_layers  # e4m3 K and V of one token
    proj = shape.n_layers * shape.d_model * (2 * shape.q_width + 2 * shape.kv_width + 3 * shape.d_ffn)
    head = shape.vocab * shape.d_model
    norms = 2 * shape.d_model * (2 * shape.n_layers + 1)
    out = {"metric": "decode tokens/s, Llama-3.3-70B shape, batch 32, context 4096, e4m3 KV, 1 GPU",
           "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "higher_is_better": True,
           "data": "synthetic (seeded N(0,0.02) bf16 weights; FP8 run: their block-scaled FP8 rounding made on "
                   "the device; uniform random tokens)",
           "config": {"workload": wl.name, "global_batch": n, "seq_len": plen}}
    for mode in ("bf16", "fp8"):
        w = dict(weights)
        if mode == "bf16":
            w["layers"] = [{k: v for k, v in lw.items() if k != "fp8"} for lw in weights["layers"]]
            w.pop("lm_head_fp8", None)
        rt = PieRuntime(shape, w, pages * page_bytes, max_rows=per_launch * plen, max_seqs=n, max_readout=n,
                        max_ctx=max_ctx)
        ws = [rt.alloc() for _ in range(n)]
        nxt = np.zeros(n, dtype=np.int32)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for b in range(0, n, per_launch):
            ss = range(b, b + per_launch)
            toks, _ = rt.forward([Pass(ws[s], wl.prompt(s), [plen - 1], [(0, 1.0, 0)]) for s in ss])
            nxt[b:b + per_launch] = toks
        torch.cuda.synchronize()
        t_pf = time.perf_counter() - t0
        ws_arr = np.array(ws, dtype=np.uint64)
        for _ in range(W):
            nxt[:] = rt.decode_step(ws_arr, nxt)
        ctx_first = rt.ws_info(ws[0])["len"] + 1
        tok_dev = torch.tensor(nxt, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            rt.decode_async(ws_arr, tok_dev, tok_dev)
        rt.sync()
        torch.cuda.synchronize()
        t_dec = time.perf_counter() - t0
        rt.close()
        ms = t_dec / K * 1e3
        wbytes = (proj + head) * (1 if mode == "fp8" else 2) + norms
        if mode == "fp8":
            wbytes += 4 * (proj + head) // (128 * 128)
        step_bytes = wbytes + sum(n * (ctx_first + i) for i in range(K)) / K * kv_tok
        out[mode] = {"value": round(n * K / t_dec, 2), "ms_per_step": round(ms, 3),
                     "context": [ctx_first, ctx_first + K - 1],
                     "step_hbm": {"bytes_per_step": int(step_bytes),
                                  "achieved_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1),
                                  "frac": round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
                     "prefill_tokens_per_s": round(n * plen / t_pf, 1)}
        log("bench 70b: %s decode %.2f ms per step, prefill %.0f tokens/s" % (mode, ms, n * plen / t_pf))
    out["value"] = out["bf16"]["value"]
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=125)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="(always on; kept for old command lines)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 outputs under DIR and exit")
    ap.add_argument("--model", default="llama31-8b", choices=["llama31-8b", "llama33-70b"],
                    help="llama33-70b: decode at the 70B shape (workload 5) with bf16 and FP8 weights")
    ap.add_argument("--no-fp8-variant", action="store_true",
                    help="skip the FP8-weight decode measured beside the headline")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="the FP8 variant: layer projections are block-scaled FP8 (e4m3 codes, one "
                         "power-of-two scale per 128 x 128 block) and decode streams the FP8 copies")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (the known-size "
                         "kernel that scales HBM byte counters) and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return
    if args.model == "llama33-70b":
        bench_70b(min(args.steps, 32), min(args.warmup, 3))
        return
    import synth
    from paged_kv_forward_amd import _native as N
    from paged_kv_forward_amd.runtime import Pass, PieRuntime, upload_weights

    torch.cuda.set_device(0)
    shape = synth.LLAMA_8B
    fp8 = args.fp8_weights
    recipe = synth.WeightRecipe(shape, fp8_blocks=fp8)
    wl = synth.workload(2)
    t0 = time.perf_counter()
    log("bench: drawing and uploading %.2f B seeded weights%s" % (shape.n_params() / 1e9,
                                                                  " (FP8 projections)" if fp8 else ""))
    weights = upload_weights(recipe, "cuda:0", progress=lambda l: (l % 8 == 7) and log("  layer", l + 1),
                             fp8=fp8)
    log("bench: weights ready in %.1f s" % (time.perf_counter() - t0))
    K, W = args.steps, args.warmup
    max_ctx = PROMPT + W + 3 * K + 3 + 8
    pages = N_SEQ * ((max_ctx + 15) // 16 + 1)
    page_bytes = shape.n_layers * 2 * shape.n_kv_heads * 16 * shape.head_dim * 2
    rt = PieRuntime(shape, weights, pages * page_bytes, max_rows=PREFILL_SEQS_PER_LAUNCH * PROMPT,
                    max_seqs=N_SEQ, max_readout=N_SEQ, max_ctx=max_ctx)
    ws = [rt.alloc() for _ in range(N_SEQ)]
    prompts = [wl.prompt(s) for s in range(N_SEQ)]

    # ---- prefill (setup) ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nxt = np.zeros(N_SEQ, dtype=np.int32)
    gemm_classes = ["gemm_qkv", "gemm_o", "gemm_gateup", "gemm_down"]
    n_launch = N_SEQ // PREFILL_SEQS_PER_LAUNCH
    t_untimed, n_untimed = None, 0
    for b in range(0, N_SEQ, PREFILL_SEQS_PER_LAUNCH):
        if b // PREFILL_SEQS_PER_LAUNCH == n_launch - PREFILL_TIMED_LAUNCHES:
            # prefill tokens/s is taken over the launches before this point:
            # the event records of the profiled ones below add gaps
            torch.cuda.synchronize()
            t_untimed, n_untimed = time.perf_counter() - t0, b
            # the last launches run with HIP events around every GEMM and
            # prefill-attention launch
            rt.profile_enable(gemm_classes + ["attn_prefill"])
        ss = range(b, b + PREFILL_SEQS_PER_LAUNCH)
        toks, _ = rt.forward([Pass(ws[s], prompts[s], [PROMPT - 1], [(0, 1.0, 0)]) for s in ss])
        nxt[b:b + PREFILL_SEQS_PER_LAUNCH] = toks
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    pf = rt.profile_read()
    rt.profile_enable([])
    log("bench: prefill %d x %d tokens in %.2f s" % (N_SEQ, PROMPT, t_prefill))
    # prefill GEMM flops per launch (T rows x 2 N K per projection, every layer)
    T_pf = PREFILL_SEQS_PER_LAUNCH * PROMPT
    d, f_, hq, hk = shape.d_model, shape.d_ffn, shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    nk_pairs = {"gemm_qkv": (hq + 2 * hk, d), "gemm_o": (d, hq), "gemm_gateup": (2 * f_, d), "gemm_down": (d, f_)}
    gemm_flop = {c: 2.0 * T_pf * n * k * shape.n_layers for c, (n, k) in nk_pairs.items()}
    gemm_ms = {c: pf[c][0] / PREFILL_TIMED_LAUNCHES for c in gemm_classes}
    tot_ms = sum(gemm_ms.values())
    tot_flop = sum(gemm_flop.values())
    prefill_gemm = {
        "bound": "mfma", "achieved": round(tot_flop / (tot_ms * 1e-3) / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(tot_flop / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops_per_launch": tot_flop, "gemm_ms_per_launch": round(tot_ms, 3),
        "by_projection_tflops": {c[5:]: round(gemm_flop[c] / (gemm_ms[c] * 1e-3) / 1e12, 1) for c in gemm_classes},
        # all layers of one prefill launch
        "attn_prefill_ms_per_launch": round(pf["attn_prefill"][0] / PREFILL_TIMED_LAUNCHES, 3),
        # causal attention: scores and P.V, 2 x 2 flops per (query, key <= query) pair per head dim
        "attn_prefill_tflops": round(4.0 * shape.n_q_heads * shape.head_dim * (PROMPT * (PROMPT + 1) / 2)
                                     * PREFILL_SEQS_PER_LAUNCH * shape.n_layers
                                     / (pf["attn_prefill"][0] / PREFILL_TIMED_LAUNCHES * 1e-3) / 1e12, 1),
        "timed_over": "the last %d prefill launches (%d rows each), HIP events around every GEMM and "
                      "prefill-attention launch" % (PREFILL_TIMED_LAUNCHES, T_pf)}

    ws_arr = np.array(ws, dtype=np.uint64)

    def step():
        nxt[:] = rt.decode_step(ws_arr, nxt)  # argmax; each sequence feeds back its own token

    for _ in range(W):
        step()
    ctx_first = rt.ws_info(ws[0])["len"] + 1
    # timed region: K loop-carried decode steps (pie_decode_async): each step
    # reads its tokens from the previous step's device output and the host
    # packs step k + 1 while the GPU runs step k; one wait at the end
    tok_dev = torch.tensor(nxt, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        rt.decode_async(ws_arr, tok_dev, tok_dev)
    rt.sync()
    torch.cuda.synchronize()
    t_dec = time.perf_counter() - t0
    log("bench: %d loop-carried decode steps in %.3f s" % (K, t_dec))
    nxt[:] = tok_dev.cpu().numpy()
    # the same K steps through the synchronous call (tokens back on the host every step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t0
    log("bench: %d host-loop decode steps in %.3f s" % (K, t_host))
    # third timed pass of K steps: HIP events on the library's stream around
    # every decode-attention launch, which runs ATTN_REPS times back to back
    # there (same inputs and outputs), so that the events' own cost (several
    # microseconds of idle GPU per interval) is shared by ATTN_REPS launches
    ctx_prof = rt.ws_info(ws[0])["len"] + 1
    rt.profile_repeat(ATTN_REPS)
    rt.profile_enable(["attn_decode"])
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    t_prof = time.perf_counter() - t0
    prof = rt.profile_read()
    rt.profile_enable([])
    rt.profile_repeat(1)

    # algorithmic bytes of decode attention: every K and V element of every
    # sequence's context once, plus q in and o out
    kv_tok = shape.n_kv_heads * shape.head_dim * 2 * 2
    qo = N_SEQ * shape.q_width * 2 * 2
    ctx_sum = sum(N_SEQ * (ctx_first + i) for i in range(K))
    ctx_sum_prof = sum(N_SEQ * (ctx_prof + i) for i in range(K))
    # over the timed pass, where each launch ran ATTN_REPS times
    attn_bytes = (ctx_sum_prof * kv_tok + K * qo) * shape.n_layers * ATTN_REPS
    attn_ms, attn_n = prof["attn_decode"]
    attn_gbs = attn_bytes / (attn_ms / 1e3) / 1e9 if attn_ms > 0 else 0.0
    per_launch = attn_bytes / max(attn_n, 1)
    weight_bytes = 2 * (shape.n_params() - shape.vocab * shape.d_model)  # all but the embedding table
    proj_params = shape.n_layers * shape.d_model * (2 * shape.q_width + 2 * shape.kv_width + 3 * shape.d_ffn)
    if fp8:  # projections and lm_head at one byte per weight plus one fp32 scale per 128 x 128 block
        f8p = proj_params + shape.vocab * shape.d_model
        weight_bytes -= f8p - 4 * f8p // (128 * 128)
    step_bytes = weight_bytes + (ctx_sum / K) * kv_tok * shape.n_layers
    ms_step = t_dec / K * 1e3

    # every kernel class of 3 more steps with HIP events: time per step, and
    # for the HBM-bound classes their algorithmic bytes per step / that time
    ctx_bd = rt.ws_info(ws[0])["len"] + 1
    rt.profile_enable(N.KERNEL_CLASSES)
    for _ in range(3):
        step()
    pb = rt.profile_read()
    rt.profile_enable([])
    breakdown = {k: round(v[0] / 3, 4) for k, v in pb.items() if v[1]}
    d, L_ = shape.d_model, shape.n_layers
    wb = 1 if fp8 else 2  # bytes per projection weight streamed by decode
    wbytes = {"gemm_qkv": wb * L_ * d * (shape.q_width + 2 * shape.kv_width),
              "gemm_o": wb * L_ * shape.q_width * d, "gemm_gateup": wb * L_ * d * 2 * shape.d_ffn,
              "gemm_down": wb * L_ * shape.d_ffn * d, "lm_head": wb * shape.vocab * d,
              "attn_decode": L_ * (sum(N_SEQ * (ctx_bd + i) for i in range(3)) / 3 * kv_tok + qo)}
    decode_kernels = {}
    for k, b in wbytes.items():
        if k in breakdown and breakdown[k] > 0:
            gbs = b / (breakdown[k] * 1e-3) / 1e9
            decode_kernels[k] = {"ms_per_step": breakdown[k], "bytes_per_step": int(b),
                                 "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}

    traffic = measured_traffic()
    out = {
        "metric": "decode tokens/s + HBM-roofline fraction, Llama-3.1-8B shape, batch 64, 1 GPU",
        "value": round(N_SEQ * K / t_dec, 2),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_host_loop": round(t_host / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, uniform random tokens)" + (
            "; layer projections rounded to block-scaled FP8 (e4m3, power-of-two scale per 128x128 block)"
            if fp8 else ""),
        "config": {"workload": "llama31-8b decode: batch 64, context %d..%d, bf16 paged KV (page 16), "
                               "argmax epilogue, loop-carried steps (pie_decode_async)%s"
                               % (ctx_first, ctx_first + K - 1,
                                  ", FP8 block-scaled projection weights streamed by decode" if fp8 else ""),
                   "global_batch": N_SEQ, "seq_len": PROMPT, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "paged decode attention (split-KV + combine)",
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": round(traffic["bytes_per_dispatch"]) if traffic else None,
                     "traffic_note": ("HBM bytes per dispatch from FETCH_SIZE + WRITE_SIZE (scaled by a "
                                      "plain copy), at context %d..%d" % tuple(traffic["context_tokens"])
                                      if traffic else "counters not taken for this kernel's sources"),
                     "bytes_per_launch": int(per_launch),
                     "avg_launch_ms": round(attn_ms / max(attn_n, 1), 5),
                     "timed_over": "a third pass of %d decode steps (context %d..%d): HIP events around "
                                   "each launch, which runs %d times back to back between them"
                                   % (K, ctx_prof, ctx_prof + K - 1, ATTN_REPS),
                     "ms_per_step_events_pass": round(t_prof / K * 1e3, 4)},
        "step_hbm": {"bytes_per_step": int(step_bytes),
                     "achieved_gbs": round(step_bytes / (ms_step / 1e3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        # the launches before the profiled ones (whose event records add gaps)
        "prefill_tokens_per_s": round(n_untimed * PROMPT / t_untimed, 1),
        "prefill_tokens_per_s_over": "%d of %d prefill launches (%d sequences of %d tokens each), before the "
                                     "profiled ones" % (n_untimed // PREFILL_SEQS_PER_LAUNCH, n_launch,
                                                        PREFILL_SEQS_PER_LAUNCH, PROMPT),
        "prefill_gemm": prefill_gemm,
    }
    out["ms_per_step_by_kernel"] = breakdown
    out["decode_kernels_hbm"] = decode_kernels
    rt.close()
    del weights
    torch.cuda.empty_cache()
    if not fp8 and not args.no_fp8_variant:
        out["fp8_weights_decode"] = fp8_decode_summary(shape, min(K, 60), min(W, 20))
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(shape, recipe)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
