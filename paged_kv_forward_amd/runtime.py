"""Python-side owner of one pie context: device buffers come from PyTorch
(plumbing only -- every step of the forward runs in the HIP library), passes
are marshalled into the C structs of include/pie.h.
"""
from __future__ import annotations

import ctypes
import itertools
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import _native as N
from ._native import check


@dataclass
class Pass:
    """One ForwardPass: new tokens of one working set, readout rows and their epilogues."""
    ws: int
    tokens: Sequence[int]
    readout: Sequence[int] = ()
    epi: Sequence[Tuple[int, float, int]] = ()   # (kind, temperature, seed) per readout row
    positions: Optional[Sequence[int]] = None
    commit: bool = True


def model_desc(shape) -> N.pie_model_desc:
    return N.pie_model_desc(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads,
                            shape.head_dim, shape.d_ffn, shape.vocab, shape.rms_eps,
                            shape.rope_theta, shape.kv_dtype, shape.page_size)


LAYER_KEYS = ["attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down"]


PACKED_KEYS = {"q", "k", "v", "o", "gate", "up", "down"}


def _struct_dtype(ctype, formats):
    """numpy dtype with the field offsets and size of a ctypes Structure."""
    names = [f for f, _ in ctype._fields_]
    return np.dtype({"names": names, "formats": [formats[f] for f in names],
                     "offsets": [getattr(ctype, f).offset for f in names],
                     "itemsize": ctypes.sizeof(ctype)})


PASS_DT = _struct_dtype(N.pie_pass, {"ws": np.uint64, "tokens": np.uint64, "positions": np.uint64,
                                      "n_tokens": np.int32, "readout": np.uint64, "n_readout": np.int32,
                                      "epi": np.uint64, "commit": np.int32})
EPI_DT = _struct_dtype(N.pie_epilogue, {"kind": np.int32, "temperature": np.float32, "seed": np.uint64})


def upload_weights(recipe, device="cuda", progress=None, fp8=False) -> Dict:
    """Draw the seeded bf16 weights of `recipe` (a synth.WeightRecipe) on the
    host and copy them to `device`, one tensor at a time through pinned
    memory.  Projections and lm_head are converted on the device to the
    library's tiled layout (pie_pack_weight) through one staging buffer, so
    the checkpoint-layout copy never exists for more than one tensor.
    fp8: also the block-scaled FP8 copy of every layer projection
    (pie_pack_weight_fp8), under layers[l]["fp8"][name] = (codes, scales),
    which PieRuntime attaches for the decode GEMMs."""
    import torch
    import synth
    shape = recipe.shape
    biggest = max(shape.vocab * shape.d_model, 3 * shape.d_model * shape.d_ffn)
    stage = torch.empty(biggest, dtype=torch.int16, pin_memory=True)
    stage_np = stage.numpy().view(np.uint16)
    dev_stage = torch.empty(max(shape.vocab * shape.d_model, shape.d_model * shape.d_ffn,
                                shape.d_model * shape.q_width), dtype=torch.int16, device=device)
    L = N.lib()

    def one(name, shp, packed=False):
        n = int(np.prod(shp))
        recipe.tensor_bits(name, shp, out=stage_np[:n])
        if not packed:
            t = torch.empty(shp, dtype=torch.bfloat16, device=device)
            t.view(torch.int16).view(-1).copy_(stage[:n], non_blocking=False)
            return t
        rows, cols = shp
        dev_stage[:n].copy_(stage[:n], non_blocking=False)
        t = torch.empty(L.pie_packed_weight_bytes(rows, cols) // 2, dtype=torch.bfloat16, device=device)
        st = torch.cuda.current_stream(device).cuda_stream
        check(L.pie_pack_weight(dev_stage.data_ptr(), t.data_ptr(), rows, cols, st))
        if fp8:
            codes = torch.empty(L.pie_packed_weight_fp8_bytes(rows, cols), dtype=torch.uint8, device=device)
            scales = torch.empty(L.pie_fp8_scale_count(rows, cols), dtype=torch.float32, device=device)
            check(L.pie_pack_weight_fp8(dev_stage.data_ptr(), codes.data_ptr(), scales.data_ptr(), rows, cols, st))
            f8[name.split(".")[-1]] = (codes, scales)
        return t

    f8 = {}
    w = {"embed": one("embed", (shape.vocab, shape.d_model)),
         "final_norm": one("final_norm", (shape.d_model,)),
         "lm_head": one("head", (shape.vocab, shape.d_model), packed=True), "layers": []}
    if fp8:
        w["lm_head_fp8"] = f8["head"]
    for l in range(shape.n_layers):
        f8 = {}
        w["layers"].append({k: one("layers.%d.%s" % (l, k), s, packed=k in PACKED_KEYS)
                            for k, s in synth.layer_tensor_shapes(shape)})
        if fp8:
            w["layers"][-1]["fp8"] = f8
        if progress:
            progress(l)
    del dev_stage
    if shape.kv_dtype == synth.KV_E4M3:
        w["kv_scale"] = torch.from_numpy(synth.kv_scales(shape)).to(device)
    return w


def torch_int32():
    import torch
    return torch.int32


class PieRuntime:
    """One context over torch-owned device memory (or a host-only context when
    weights is None: working sets and packing without the GPU)."""

    def __init__(self, shape, weights: Optional[Dict], kv_bytes: int, max_rows: int,
                 max_seqs: int, max_readout: int, max_ctx: int, device="cuda", stream=None,
                 workspace: bool = True):
        """workspace=False: no device workspace (pie_init with NULL, 0); the
        context then runs only forward_static (the library's static scratch)."""
        self.shape = shape
        self.desc = model_desc(shape)
        self.limits = N.pie_limits(max_rows, max_seqs, max_readout, max_ctx)
        self._keep = []
        self._decode_bufs = {}
        L = N.lib()
        self.page_bytes = L.pie_kv_page_bytes(ctypes.byref(self.desc))
        self.ws_bytes = L.pie_workspace_bytes(ctypes.byref(self.desc), ctypes.byref(self.limits))
        if self.page_bytes == 0 or self.ws_bytes == 0:
            raise N.PieError(N.PIE_EINVAL, "bad model shape or limits")
        ctx = ctypes.c_void_p()
        if weights is None:
            check(L.pie_init(ctypes.byref(self.desc), None, None, kv_bytes, None, 0,
                             ctypes.byref(self.limits), None, ctypes.byref(ctx)))
            self.kv = self.workspace = None
            self.stream = None
        else:
            import torch
            self.device = torch.device(device)
            self.kv = torch.empty(kv_bytes, dtype=torch.uint8, device=self.device)
            self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
                              if workspace else None)
            self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
            self.weights = weights
            pw = self._weights_struct(weights)
            check(L.pie_init(ctypes.byref(self.desc), ctypes.byref(pw), self.kv.data_ptr(), kv_bytes,
                             self.workspace.data_ptr() if workspace else None, self.ws_bytes if workspace else 0,
                             ctypes.byref(self.limits), ctypes.c_void_p(self.stream.cuda_stream),
                             ctypes.byref(ctx)))
            if "fp8" in weights["layers"][0]:
                check(L.pie_attach_fp8_weights(ctx, ctypes.byref(self._fp8_struct(weights))))
        self.ctx = ctx

    def _fp8_struct(self, w):
        L = self.shape.n_layers
        fields = []
        for i in (0, 1):  # codes, then scales
            for k in ("q", "k", "v", "o", "gate", "up", "down"):
                fields.append((ctypes.c_void_p * L)(*[w["layers"][l]["fp8"][k][i].data_ptr() for l in range(L)]))
        self._keep.append(fields)
        head = w.get("lm_head_fp8")
        return N.pie_fp8_weights(*fields, head[0].data_ptr() if head else None,
                                 head[1].data_ptr() if head else None)

    def _weights_struct(self, w):
        L = self.shape.n_layers
        arrs = {}
        for k in LAYER_KEYS:
            a = (ctypes.c_void_p * L)(*[w["layers"][l][k].data_ptr() for l in range(L)])
            arrs[k] = a
        self._keep.append(arrs)
        ks = w.get("kv_scale")
        return N.pie_weights(w["embed"].data_ptr(), w["final_norm"].data_ptr(),
                             w["lm_head"].data_ptr(), arrs["attn_norm"], arrs["q"], arrs["k"],
                             arrs["v"], arrs["o"], arrs["mlp_norm"], arrs["gate"], arrs["up"],
                             arrs["down"], ks.data_ptr() if ks is not None else None)

    # ------------------------------------------------------------ working sets
    def alloc(self) -> int:
        h = ctypes.c_uint64()
        check(N.lib().pie_alloc_working_set(self.ctx, ctypes.byref(h)))
        return h.value

    def fork(self, parent: int) -> int:
        h = ctypes.c_uint64()
        check(N.lib().pie_fork(self.ctx, parent, ctypes.byref(h)))
        return h.value

    def free(self, ws: int) -> None:
        check(N.lib().pie_free_working_set(self.ctx, ws))

    def truncate(self, ws: int, new_len: int) -> None:
        check(N.lib().pie_truncate(self.ctx, ws, new_len))

    def ws_info(self, ws: int):
        st = N.pie_ws_stats()
        check(N.lib().pie_ws_info(self.ctx, ws, ctypes.byref(st), None))
        ids = (ctypes.c_int32 * max(st.n_pages, 1))()
        check(N.lib().pie_ws_info(self.ctx, ws, ctypes.byref(st), ids))
        return {"len": st.len, "frozen_len": st.frozen_len,
                "pages": np.frombuffer(ids, dtype=np.int32)[:st.n_pages].copy()}

    def pool_stats(self) -> Dict[str, int]:
        st = N.pie_pool_stats()
        check(N.lib().pie_pool_stats_get(self.ctx, ctypes.byref(st)))
        return {k: getattr(st, k) for k, _ in N.pie_pool_stats._fields_}

    # ------------------------------------------------------------ forward
    def _marshal(self, passes: Sequence[Pass]):
        """The pie_pass array of `passes`, built with a few numpy operations: all
        tokens, positions, readout indices and epilogues of the call sit in one
        array each, and each pass points into them."""
        n = len(passes)
        chain = itertools.chain.from_iterable
        n_tok = np.fromiter((len(p.tokens) for p in passes), dtype=np.int64, count=n)
        if n_tok.sum() <= 4096 and not any(isinstance(p.tokens, np.ndarray) for p in passes):
            tok = np.fromiter(chain(p.tokens for p in passes), dtype=np.int32, count=int(n_tok.sum()))
        else:
            tok = np.concatenate([np.asarray(p.tokens, dtype=np.int32).reshape(-1) for p in passes])
        n_ro = np.fromiter((len(p.readout) for p in passes), dtype=np.int64, count=n)
        R = int(n_ro.sum())
        ro = np.fromiter(chain(p.readout for p in passes), dtype=np.int32, count=R) if R else np.zeros(1, np.int32)
        epi = np.zeros(max(R, 1), dtype=EPI_DT)
        if R:
            epis = list(chain(p.epi for p in passes))
            epi["kind"] = np.fromiter((e[0] for e in epis), dtype=np.int32, count=R)
            epi["temperature"] = np.fromiter((e[1] for e in epis), dtype=np.float32, count=R)
            epi["seed"] = np.fromiter((int(e[2]) & 0xFFFFFFFFFFFFFFFF for e in epis), dtype=np.uint64, count=R)
        has_pos = np.fromiter((p.positions is not None for p in passes), dtype=bool, count=n)
        pos = None
        if has_pos.any():
            pos = np.concatenate([np.asarray(p.positions if p.positions is not None else np.zeros(len(p.tokens)),
                                             dtype=np.int32).reshape(-1) for p in passes])
        tok_off = np.zeros(n, dtype=np.uint64)
        np.cumsum(n_tok[:-1], out=tok_off[1:])
        ro_off = np.zeros(n, dtype=np.uint64)
        np.cumsum(n_ro[:-1], out=ro_off[1:])
        arr = np.zeros(n, dtype=PASS_DT)
        arr["ws"] = np.fromiter((p.ws for p in passes), dtype=np.uint64, count=n)
        arr["tokens"] = np.uint64(tok.ctypes.data) + tok_off * np.uint64(4)
        if pos is not None:
            arr["positions"] = np.where(has_pos, np.uint64(pos.ctypes.data) + tok_off * np.uint64(4), np.uint64(0))
        arr["n_tokens"] = n_tok
        arr["readout"] = np.where(n_ro > 0, np.uint64(ro.ctypes.data) + ro_off * np.uint64(4), np.uint64(0))
        arr["n_readout"] = n_ro
        arr["epi"] = np.where(n_ro > 0, np.uint64(epi.ctypes.data) + ro_off * np.uint64(EPI_DT.itemsize),
                              np.uint64(0))
        arr["commit"] = np.fromiter((p.commit for p in passes), dtype=np.int32, count=n)
        return arr, [tok, ro, epi, pos, arr]

    def decode_step(self, ws: np.ndarray, tokens: np.ndarray, kind=0, temperature=1.0, seed=0,
                    flags: int = 0, logits_out=None) -> np.ndarray:
        """One decode token for each working set in `ws` (uint64 handles), read
        out with the given epilogue (scalars or per-row arrays); committed.
        The same pie_forward call as forward(), with the pass array built by
        vector operations on buffers reused across calls of the same batch size.
        Returns the token ids (int32)."""
        n = len(ws)
        buf = self._decode_bufs.get(n)
        if buf is None:
            arr = np.zeros(n, dtype=PASS_DT)
            tok = np.zeros(n, dtype=np.int32)
            ro = np.zeros(n, dtype=np.int32)
            epi = np.zeros(n, dtype=EPI_DT)
            out = np.zeros(n, dtype=np.int32)
            idx = np.arange(n, dtype=np.uint64)
            arr["tokens"] = np.uint64(tok.ctypes.data) + idx * np.uint64(4)
            arr["n_tokens"] = 1
            arr["readout"] = np.uint64(ro.ctypes.data)  # every pass reads out its only row
            arr["n_readout"] = 1
            arr["epi"] = np.uint64(epi.ctypes.data) + idx * np.uint64(EPI_DT.itemsize)
            arr["commit"] = 1
            # every array the pass records point into is kept alive with them
            buf = self._decode_bufs[n] = (arr, tok, epi, out, ro)
        arr, tok, epi, out, _ = buf
        arr["ws"] = ws
        tok[:] = tokens
        epi["kind"] = kind
        epi["temperature"] = temperature
        epi["seed"] = seed
        logits_ptr = None
        if logits_out is not None:
            logits_ptr = logits_out.data_ptr()
            flags |= N.PIE_FLAG_LOGITS_DEVICE
        check(N.lib().pie_forward(self.ctx, arr.ctypes.data_as(ctypes.POINTER(N.pie_pass)), n,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), logits_ptr, flags))
        return out.copy()

    def decode_async(self, ws: np.ndarray, tokens_in, tokens_out, kind=0, temperature=1.0, seed=0,
                     logits_out=None) -> None:
        """Enqueue one loop-carried decode step (pie_decode_async): one token per
        working set in `ws` (uint64 handles), read from the device int32 tensor
        `tokens_in`, the chosen tokens written to the device int32 tensor
        `tokens_out` (which may be `tokens_in`); returns without waiting.
        Epilogue parameters are scalars or per-row arrays."""
        n = len(ws)
        for t in (tokens_in, tokens_out):
            if t.dtype != torch_int32() or not t.is_cuda or t.numel() < n or not t.is_contiguous():
                raise ValueError("tokens_in / tokens_out: contiguous int32 device tensors of >= %d elements" % n)
        key = ("async", n)
        buf = self._decode_bufs.get(key)
        if buf is None:
            buf = self._decode_bufs[key] = (np.zeros(n, dtype=np.uint64), np.zeros(n, dtype=EPI_DT))
        wsa, epi = buf
        wsa[:] = ws
        epi["kind"] = kind
        epi["temperature"] = temperature
        epi["seed"] = seed
        check(N.lib().pie_decode_async(
            self.ctx, wsa.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n, tokens_in.data_ptr(),
            tokens_out.data_ptr(), epi.ctypes.data_as(ctypes.POINTER(N.pie_epilogue)),
            logits_out.data_ptr() if logits_out is not None else None))

    def prefix_lookup(self, tokens) -> Tuple[int, int]:
        """(working set, shared length): a new working set holding the longest
        remembered page-aligned prefix of `tokens` (pie_prefix_lookup)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        h = ctypes.c_uint64()
        k = ctypes.c_int32()
        check(N.lib().pie_prefix_lookup(self.ctx, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(t),
                                        ctypes.byref(h), ctypes.byref(k)))
        return h.value, k.value

    def sync(self) -> None:
        """Wait for every enqueued step (pie_sync)."""
        check(N.lib().pie_sync(self.ctx))

    def forward_static(self, passes: Sequence[Pass], want_logits: bool = False, flags: int = 0,
                       logits_out=None):
        """pie_forward_static: as forward, over the library's static device scratch."""
        return self.forward(passes, want_logits, flags, logits_out, _entry="pie_forward_static")

    def forward(self, passes: Sequence[Pass], want_logits: bool = False, flags: int = 0,
                logits_out=None, _entry: str = "pie_forward"):
        """Returns (tokens int32[R], logits float32[R, V] or None)."""
        arr, keep = self._marshal(passes)
        if os.environ.get("PIE_SYNC_DEBUG"):
            flags |= N.PIE_FLAG_SYNC_DEBUG
        R = sum(len(p.readout) for p in passes)
        toks = np.full(max(R, 1), -1, dtype=np.int32)
        logits_ptr = None
        logits = None
        if logits_out is not None:
            logits_ptr = logits_out.data_ptr()
            flags |= N.PIE_FLAG_LOGITS_DEVICE
            logits = logits_out
        elif want_logits and R:
            logits = np.empty((R, self.shape.vocab), dtype=np.float32)
            logits_ptr = logits.ctypes.data
        check(getattr(N.lib(), _entry)(self.ctx, arr.ctypes.data_as(ctypes.POINTER(N.pie_pass)), len(passes),
                                       toks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       logits_ptr, flags))
        del keep
        return toks[:R], logits

    def plan(self) -> Dict[str, np.ndarray]:
        v = N.pie_plan_view()
        check(N.lib().pie_debug_plan(self.ctx, ctypes.byref(v)))
        sizes = {"tok": v.n_rows, "pos": v.n_rows, "row_seq": v.n_rows, "slot": v.n_rows,
                 "seq_row0": v.n_seqs + 1, "seq_ctx": v.n_seqs, "seq_len": v.n_seqs,
                 "seq_pg0": v.n_seqs + 1, "pg_id": v.n_page_entries,
                 "pg_valid": v.n_page_entries, "pg_start": v.n_page_entries,
                 "ro_row": v.n_readout, "ro_lane": v.n_readout}
        out = {}
        for k, n in sizes.items():
            ptr = getattr(v, k)
            out[k] = np.ctypeslib.as_array(ptr, shape=(n,)).copy() if n else np.zeros(0, np.int32)
        return out

    # ------------------------------------------------------------ measurement
    def profile_enable(self, classes: Sequence[str]) -> None:
        mask = 0
        for c in classes:
            mask |= 1 << N.KERNEL_CLASSES.index(c)
        check(N.lib().pie_profile_enable(self.ctx, mask))

    def profile_repeat(self, reps: int) -> None:
        """Timed decode-attention launches run reps times back to back."""
        check(N.lib().pie_profile_repeat(self.ctx, int(reps)))

    def profile_read(self) -> Dict[str, Tuple[float, int]]:
        ms = (ctypes.c_double * N.PIE_K_NUM_CLASSES)()
        cnt = (ctypes.c_int64 * N.PIE_K_NUM_CLASSES)()
        check(N.lib().pie_profile_read(self.ctx, ms, cnt))
        return {c: (ms[i], cnt[i]) for i, c in enumerate(N.KERNEL_CLASSES)}

    def philox(self, seed: int, lane: int, v0: int, n: int) -> np.ndarray:
        import torch
        out = torch.empty(n, dtype=torch.int32, device=self.device)
        check(N.lib().pie_debug_philox(self.ctx, seed & 0xFFFFFFFFFFFFFFFF, lane, v0, n,
                                       out.data_ptr()))
        return out.cpu().numpy().view(np.uint32)

    def close(self):
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            N.lib().pie_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
