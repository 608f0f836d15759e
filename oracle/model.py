"""The Llama-style decoder of the pages, one plain function per step.
Test infrastructure only.

The graph is the Poem forward of "Write a model in Poem", §5 Forward pass:
embed the tokens; per layer, x = rmsnorm(y, attn_norm), y = y + attention(x),
x = rmsnorm(y, mlp_norm), y = y + swiglu(x); then rmsnorm(y, final_norm),
gather the readout rows, lm_head.  The bodies of the attention and swiglu
blocks are not on the pages (they are loaded from a shared library of blocks,
same page, "Shared building blocks"); this build reads them as the standard
Llama blocks: separate q/k/v/o projections without bias, rotate-half RoPE
without frequency scaling, grouped-query attention with scale 1/sqrt(head_dim)
and a causal mask in append order, and down(silu(gate x) * up x).

Numerics: float64 arithmetic.  Storage points mirror the GPU path unless
``exact``: bf16 for every matmul input (normed activations, attention output,
SwiGLU product), bf16 for q after RoPE, the KV dtype for stored K and V, and
float32 for the residual stream and the logits.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

from .numerics import round_bf16, round_f32, store_e4m3

KV_BF16 = 0
KV_E4M3 = 1


@dataclass(frozen=True)
class Numerics:
    exact: bool = False
    kv_dtype: int = KV_BF16
    kv_scales: Optional[np.ndarray] = None   # [L][2][n_kv_heads] float32, e4m3 only

    def act(self, x):
        """A value the GPU stores as bf16 before a matmul."""
        return np.asarray(x, dtype=np.float64) if self.exact else round_bf16(x)

    def resid(self, x):
        """A value the GPU stores as float32 (residual stream, logits)."""
        return np.asarray(x, dtype=np.float64) if self.exact else round_f32(x)

    def kv(self, x, layer: int, which: int):
        """Stored K (which=0) or V (which=1): x has shape [n, n_kv_heads, head_dim]."""
        if self.exact:
            return np.asarray(x, dtype=np.float64)
        if self.kv_dtype == KV_BF16:
            return round_bf16(x)
        s = self.kv_scales[layer, which]          # [n_kv_heads]
        out = np.empty(x.shape, dtype=np.float64)
        for h in range(x.shape[1]):
            out[:, h, :] = store_e4m3(x[:, h, :], float(s[h]))
        return out


# ----------------------------------------------------------------------------
# Steps
# ----------------------------------------------------------------------------

def rmsnorm(y: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """ops.elemwise.rmsnorm (Poem ops, "Operations"; used in §5 Forward pass):
    y / sqrt(mean(y^2) + eps) * g over the last axis."""
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """ops.elemwise.rope, rotate-half convention.  x: [n, heads, hd]; pos: [n].

    For j < hd/2 the pair (x_j, x_{j+hd/2}) is rotated by the angle
    pos * theta^(-2j/hd), angles in float64.  The pairing is a reading: the
    pages give only the op's name.
    """
    n, _, hd = x.shape
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_ctx: int) -> np.ndarray:
    """ops.attn.attend / ops.attn.prefill: grouped-query causal attention.

    q: [n, nq, hd] new rows; K, V: [n_ctx + n, nkv, hd] in append order, the
    first n_ctx entries being the cached context.  New row i sees entries
    0 .. n_ctx + i.  Query head h reads KV head h // (nq / nkv).  Scores are
    scaled by 1/sqrt(hd); softmax subtracts the row maximum.  Returns [n, nq, hd].
    """
    n, nq, hd = q.shape
    nkv = K.shape[1]
    group = nq // nkv
    total = K.shape[0]
    assert total == n_ctx + n
    visible = np.arange(total)[None, :] <= (n_ctx + np.arange(n))[:, None]
    out = np.empty((n, nq, hd), dtype=np.float64)
    for h in range(nq):
        kv = h // group
        s = (q[:, h, :] @ K[:, kv, :].T) / np.sqrt(hd)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, kv, :]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    """ops.elemwise.silu: x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def matmul_t(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """ops.linear.matmul with a checkpoint-layout weight: a @ w.T, float64."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


# ----------------------------------------------------------------------------
# One decoder layer and the head
# ----------------------------------------------------------------------------

def layer_forward(lw: Dict[str, np.ndarray], h: np.ndarray, pos: np.ndarray,
                  K_ctx: np.ndarray, V_ctx: np.ndarray, shape, num: Numerics, layer: int
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """block(l, w, y) of §5 Forward pass for n new rows of one sequence.

    h: [n, d] residual stream of the new rows; K_ctx, V_ctx: [n_ctx, nkv, hd]
    stored K/V of the sequence's earlier tokens at this layer.  Returns the new
    residual rows and the stored K, V of the new rows.
    """
    n = h.shape[0]
    nq, nkv, hd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    # x = rmsnorm(y, attn_norm)
    a = num.act(rmsnorm(h, lw["attn_norm"], shape.rms_eps))
    # attention(x, ..., positions)
    q = matmul_t(a, lw["q"]).reshape(n, nq, hd)
    k = matmul_t(a, lw["k"]).reshape(n, nkv, hd)
    v = matmul_t(a, lw["v"]).reshape(n, nkv, hd)
    q = num.act(rope(q, pos, shape.rope_theta))
    k = rope(k, pos, shape.rope_theta)
    K_new = num.kv(k, layer, 0)
    V_new = num.kv(v, layer, 1)
    K = np.concatenate([K_ctx, K_new], axis=0)
    V = np.concatenate([V_ctx, V_new], axis=0)
    o = num.act(attention(q, K, V, K_ctx.shape[0]).reshape(n, nq * hd))
    # y = residual_add(attention(...), y)
    h = num.resid(h + matmul_t(o, lw["o"]))
    # x = rmsnorm(y, mlp_norm); y = residual_add(swiglu(x), y)
    m = num.act(rmsnorm(h, lw["mlp_norm"], shape.rms_eps))
    z = num.act(silu(matmul_t(m, lw["gate"])) * matmul_t(m, lw["up"]))
    h = num.resid(h + matmul_t(z, lw["down"]))
    return h, K_new, V_new


def head_logits(h_rows: np.ndarray, final_norm: np.ndarray, head: np.ndarray, shape,
                num: Numerics) -> np.ndarray:
    """rmsnorm(y, final_norm) -> gather_rows -> lm_head for rows already gathered
    (the norm is row-wise, so gathering first gives the same rows).  Logits are
    held in float32 by the GPU: returned as float64 (``exact``) or rounded."""
    x = num.act(rmsnorm(h_rows, final_norm, shape.rms_eps))
    return num.resid(matmul_t(x, head))
