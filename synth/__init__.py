"""Seeded synthetic inputs shared by the HIP path's harness and the oracle.

This module holds the model shapes of the workloads, and turns seeds into
weights, prompt tokens, context lengths, epilogue choices and KV scales.  It
holds none of the forward pass's arithmetic: the numbers come from the
counter-based generator in ``synth.c`` (SplitMix64 + Box-Muller, see there),
which both sides call, so the GPU harness and the oracle see the same bytes.

Weights follow the usual random init of the workloads: every matrix and the
embedding are N(0, 0.02) rounded to bf16, and norm gains are 1.0 unless a
gain spread is asked for (then N(1, gain_std), rounded to bf16).
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build_lib(force: bool = False) -> str:
    """Compile synth.c into libsynth.so with gcc (OpenMP for the bulk fills)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_at.restype = ctypes.c_uint64
        lib.synth_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal_at.restype = ctypes.c_double
        lib.synth_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_int]
        lib.synth_uniform_int.restype = None
        lib.synth_uniform_int.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32]
        lib.synth_uniform_f64.restype = None
        lib.synth_uniform_f64.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64]
        _lib = lib
    return _lib


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n) or n)))


def key_of(text: str) -> int:
    """64-bit key = first 8 bytes (little endian) of SHA-256(text)."""
    return int.from_bytes(hashlib.sha256(text.encode()).digest()[:8], "little")


def normal_bf16(n: int, key: int, mean: float = 0.0, std: float = 0.02, first: int = 0,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    """n bf16 values (as uint16 bit patterns) of mean + std * N(0,1) from stream `key`."""
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    if n:
        _load().synth_normal_bf16(out.ctypes.data, n, key, first, mean, std, n_threads())
    return out


def uniform_int(n: int, key: int, lo: int, hi: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _load().synth_uniform_int(out.ctypes.data, n, key, first, lo, hi)
    return out


def uniform_f64(n: int, key: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_uniform_f64(out.ctypes.data, n, key, first)
    return out


def raw_u64(key: int, i: int) -> int:
    return int(_load().synth_at(key, i))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Model shapes
# ----------------------------------------------------------------------------

KV_BF16 = 0
KV_E4M3 = 1


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0
    kv_dtype: int = KV_BF16
    page_size: int = 16

    @property
    def q_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def n_params(self) -> int:
        d, f = self.d_model, self.d_ffn
        per_layer = 2 * d + d * (self.q_width + 2 * self.kv_width) + self.q_width * d + 3 * d * f
        return 2 * self.vocab * d + d + self.n_layers * per_layer


TINY = ModelShape("tiny-2l", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                  d_ffn=688, vocab=4096)
LLAMA_8B = ModelShape("llama31-8b", n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8,
                      head_dim=128, d_ffn=14336, vocab=128256)
LLAMA_70B = ModelShape("llama33-70b", n_layers=80, d_model=8192, n_q_heads=64, n_kv_heads=8,
                       head_dim=128, d_ffn=28672, vocab=128256, kv_dtype=KV_E4M3)

SHAPES = {s.name: s for s in (TINY, LLAMA_8B, LLAMA_70B)}


def first_layers(shape: ModelShape, n_layers: int) -> ModelShape:
    """The same model cut to its first n_layers layers (weights are drawn by
    tensor name, so the kept layers, embedding and head are identical)."""
    return replace(shape, name="%s-first%d" % (shape.name, n_layers), n_layers=n_layers)


FP8_BLOCK = 128
E4M3_MAX = 448.0


def fp8_block_bits(bits: np.ndarray) -> np.ndarray:
    """A weight matrix drawn for a block-scaled FP8 model: each 128 x 128 block
    of the [out][in] bf16 matrix `bits` becomes the nearest OCP e4m3 values
    (ties to even, saturating at 448) times the block's power-of-two scale
    2^e, e the least integer with max |w| <= 448 * 2^e.  The result holds bf16
    bits; every value is exactly representable (at most 4 significant bits).
    This shapes an input; the forward pass only ever sees the values."""
    import torch
    rows, cols = bits.shape
    pr, pc = -(-rows // FP8_BLOCK) * FP8_BLOCK, -(-cols // FP8_BLOCK) * FP8_BLOCK
    w = torch.zeros((pr, pc), dtype=torch.float32)
    w[:rows, :cols] = (torch.from_numpy(bits.astype(np.int32)) << 16).view(torch.float32)
    blk = w.view(pr // FP8_BLOCK, FP8_BLOCK, pc // FP8_BLOCK, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3)).double()
    e = torch.where(amax > 0, torch.ceil(torch.log2(torch.where(amax > 0, amax, 1.0) / E4M3_MAX)), 0.0)
    # exact adjustment: least e with amax <= 448 * 2^e
    e = torch.where(amax > E4M3_MAX * torch.exp2(e), e + 1, e)
    e = torch.where((amax > 0) & (amax <= E4M3_MAX * torch.exp2(e - 1)), e - 1, e)
    scale = torch.exp2(e).float()[:, None, :, None]
    q = torch.clamp(blk / scale, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).float()
    out = (q * scale).reshape(pr, pc)[:rows, :cols].contiguous()
    return (out.view(torch.int32) >> 16).to(torch.int32).numpy().astype(np.uint16)


def layer_tensor_shapes(m: ModelShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """Per-layer weights, row-major [out][in] for matrices (the checkpoint layout)."""
    d, f = m.d_model, m.d_ffn
    return [("attn_norm", (d,)), ("q", (m.q_width, d)), ("k", (m.kv_width, d)),
            ("v", (m.kv_width, d)), ("o", (d, m.q_width)), ("mlp_norm", (d,)),
            ("gate", (f, d)), ("up", (f, d)), ("down", (d, f))]


@dataclass(frozen=True)
class WeightRecipe:
    """How the seeded weights of one model are drawn.  fp8_blocks: every layer
    projection and the lm_head are block-scaled FP8 matrices (see
    fp8_block_bits); their bf16 values are exactly the codes times their block
    scales.  The embedding and the norm gains stay as drawn."""
    shape: ModelShape
    weight_seed: int = 1234
    std: float = 0.02
    gain_std: float = 0.0  # 0 -> gains are exactly 1.0
    fp8_blocks: bool = False

    def key(self, name: str) -> int:
        return key_of("%d/%s" % (self.weight_seed, name))

    def tensor_bits(self, name: str, shape: Tuple[int, ...],
                    out: Optional[np.ndarray] = None) -> np.ndarray:
        n = int(np.prod(shape))
        if name.endswith("norm"):
            if self.gain_std == 0.0:
                bits = out if out is not None else np.empty(n, dtype=np.uint16)
                bits.reshape(-1)[:] = 0x3F80  # bf16(1.0)
                return bits.reshape(shape)
            return normal_bf16(n, self.key(name), 1.0, self.gain_std, out=out).reshape(shape)
        bits = normal_bf16(n, self.key(name), 0.0, self.std, out=out).reshape(shape)
        if self.fp8_blocks and (name.startswith("layers.") or name == "head"):
            bits[...] = fp8_block_bits(bits)
        return bits

    def embed_bits(self) -> np.ndarray:
        m = self.shape
        return self.tensor_bits("embed", (m.vocab, m.d_model))

    def head_bits(self) -> np.ndarray:
        m = self.shape
        return self.tensor_bits("head", (m.vocab, m.d_model))

    def final_norm_bits(self) -> np.ndarray:
        return self.tensor_bits("final_norm", (self.shape.d_model,))

    def layer_bits(self, layer: int) -> Dict[str, np.ndarray]:
        return {nm: self.tensor_bits("layers.%d.%s" % (layer, nm), shp)
                for nm, shp in layer_tensor_shapes(self.shape)}

    def embed_rows_bits(self, rows: np.ndarray) -> np.ndarray:
        """Selected embedding rows without drawing the whole table."""
        m = self.shape
        key = self.key("embed")
        out = np.empty((len(rows), m.d_model), dtype=np.uint16)
        for i, r in enumerate(np.asarray(rows, dtype=np.int64)):
            normal_bf16(m.d_model, key, 0.0, self.std, first=int(r) * m.d_model, out=out[i])
        return out


def kv_scales(m: ModelShape, seed: int = 77) -> np.ndarray:
    """Static e4m3 dequantisation scales [L][2 (K,V)][n_kv_heads], float32.

    s = 8 * std_kv / 448 * (1 + 0.25 u), u ~ U[0,1) per (layer, K|V, head), where
    std_kv = 0.02 * sqrt(d_model) is the spread of a K or V entry at the random
    init (unit-RMS normed input times N(0, 0.02) weights).  Distinct per head so
    that a kernel which mixes up heads or K/V scales is caught.
    """
    u = uniform_f64(m.n_layers * 2 * m.n_kv_heads, key_of("kv_scales/%d" % seed))
    base = 8.0 * 0.02 * np.sqrt(m.d_model) / 448.0
    return (base * (1.0 + 0.25 * u)).astype(np.float32).reshape(m.n_layers, 2, m.n_kv_heads)


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

EPI_ARGMAX = 0
EPI_GUMBEL = 1


def prompt_tokens(config_id: int, seq_id: int, n: int, vocab: int, salt: int = 7) -> np.ndarray:
    """Uniform random prompt tokens for sequence `seq_id` of workload `config_id`."""
    return uniform_int(n, key_of("tokens/%d/%d/%d" % (config_id, seq_id, salt)), 0, vocab)


def teacher_tokens(config_id: int, seq_id: int, n: int, vocab: int) -> np.ndarray:
    """Seeded tokens fed to decode steps of parity runs (instead of the model's own
    choice), so that a whole trajectory is known in advance."""
    return prompt_tokens(config_id, 1000 + seq_id, n, vocab, salt=11)


def epilogue_seed(branch_seed: int, step: int) -> int:
    """Fresh 64-bit seed per pass: (branch_seed << 32) | step."""
    return ((branch_seed & 0xFFFFFFFF) << 32) | (step & 0xFFFFFFFF)


@dataclass
class Workload:
    """A seeded workload: model shape + per-sequence prompts and decode plan."""
    config_id: int
    name: str
    shape: ModelShape
    n_seqs: int
    prompt_len: List[int]
    decode_steps: int
    epi_kind: List[int]
    temperature: List[float]
    branch_seed: List[int]
    chunk: int = 0                # 0 = whole prompt in one pass
    fork_prefix: int = 0          # >0: one shared prefix of this length, forked n_seqs times
    notes: str = ""

    def prompt(self, s: int) -> np.ndarray:
        return prompt_tokens(self.config_id, s, self.prompt_len[s], self.shape.vocab)

    def prefix(self) -> np.ndarray:
        return prompt_tokens(self.config_id, 10_000, self.fork_prefix, self.shape.vocab)


def workload(config_id: int, shape: Optional[ModelShape] = None) -> Workload:
    """The five workloads, by number (1 tiny, 2 8B decode, 3 fork, 4 mix, 5 70B decode)."""
    if config_id == 1:
        m = shape or TINY
        return Workload(1, "tiny-2l: 4 seqs x 32 prompt, 8 argmax decode steps", m, 4,
                        [32] * 4, 8, [EPI_ARGMAX] * 4, [1.0] * 4, [0] * 4)
    if config_id == 2:
        m = shape or LLAMA_8B
        return Workload(2, "llama31-8b decode: batch 64, context 2048, argmax, 128 steps", m, 64,
                        [2048] * 64, 128, [EPI_ARGMAX] * 64, [1.0] * 64, [0] * 64)
    if config_id == 3:
        m = shape or LLAMA_8B
        return Workload(3, "llama31-8b fork: 8192 prefix, 10 x 256 suffix, 64 gumbel steps T=0.7",
                        m, 10, [256] * 10, 64, [EPI_GUMBEL] * 10, [0.7] * 10,
                        [0x5EED0000 + b for b in range(10)], fork_prefix=8192)
    if config_id == 4:
        m = shape or LLAMA_8B
        n_dec = 120
        ctx = uniform_int(n_dec, key_of("mix/ctx"), 128, 8193)
        kinds = uniform_int(8 + n_dec, key_of("mix/epi"), 0, 2)
        lens = [4096] * 8 + [int(c) for c in ctx]
        return Workload(4, "llama31-8b mix: 8 x 4096 prompts in 512 chunks + 120 decode rows", m,
                        8 + n_dec, lens, 8, [int(k) for k in kinds], [1.0] * (8 + n_dec),
                        [0x313C0000 + s for s in range(8 + n_dec)], chunk=512)
    if config_id == 5:
        m = shape or LLAMA_70B
        return Workload(5, "llama33-70b decode: batch 32, context 4096, e4m3 KV, argmax", m, 32,
                        [4096] * 32, 32, [EPI_ARGMAX] * 32, [1.0] * 32, [0] * 32)
    raise ValueError("unknown workload %r" % config_id)
