"""CPU oracle for the attention half of a Maple-Preview-shaped layer.

TEST INFRASTRUCTURE (like the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it;
the GPU library shares no code with it.

What the pages fix (ai.thesatyajit.com, "The architecture around the
quantization"; jj-blog, architecture list):
* the layer pattern: three sliding-window layers, then one global layer,
  repeated six times (global at layers 3, 7, 11, 15, 19, 23);
* sliding layers see a 512-token window and carry position through rotary
  embeddings on half of the head dimension (partial rotary factor 0.5);
* global layers see the whole prefix and use no positional encoding.
And the census (ai.thesatyajit.com, "The 5.31 GB claim reconciles"): 19.58B
ternary parameters, of which the experts hold 24 x 256 x 3 x 512 x 2048; the
remaining ~0.25B are the ternary attention projections, 10,485,760 per layer
= 2 x 2048 x 2048 (query, output) + 2 x 512 x 2048 (key, value).

Readings where the pages are silent (each one stated, none printed there):
head_dim 128, so 16 query heads and 4 key/value heads (query head h reads
key/value head h // 4); rotary on the first 64 dimensions of each head with
the rotate-half pairing (i, i + 32), inverse frequencies base^(-2i/64), base
10000; a sliding query at position p sees keys j with p - 512 < j <= p, a
global one every j <= p; scores scaled by 1/sqrt(128); softmax and all
intermediates in float64; no normalisation layers (their placement is not
given); output o = To (attention), residual bf16(fp32(x) + fp32(o)).

Everything is computed plainly: float64 matrix products (a library
primitive), explicit masks, an explicit softmax, no blocking or fusion.
"""
from __future__ import annotations

import numpy as np

from .tmoe_oracle import bf16_to_f64

HIDDEN = 2048
N_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 128
ROTARY_DIM = 64  # partial rotary factor 0.5 of the head dimension
WINDOW = 512
ROPE_BASE = 10000.0
N_LAYERS = 24


def is_global_layer(layer: int) -> bool:
    """Layer pattern s s s G repeated: global attention at layers 3, 7, ..., 23."""
    return layer % 4 == 3


def rope(x: np.ndarray, pos: np.ndarray, rot_dim: int = ROTARY_DIM, base: float = ROPE_BASE) -> np.ndarray:
    """Rotary position embedding on the first rot_dim dimensions of each head.

    x [..., P, d] float64, pos [P] integer positions. Pair (i, i + rot_dim/2)
    of position p turns by the angle p * base^(-2i/rot_dim); dimensions past
    rot_dim are left as they are."""
    half = rot_dim // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / rot_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    out = np.array(x, dtype=np.float64, copy=True)
    x1, x2 = x[..., :half], x[..., half:rot_dim]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rot_dim] = x2 * c + x1 * s
    return out


def visible(p: int, j: int, window: int) -> bool:
    """Key position j is visible to the query at position p (window 0: global)."""
    return j <= p and (window == 0 or p - j < window)


def attention_half(x_bits: np.ndarray, Wq: np.ndarray, Wk: np.ndarray, Wv: np.ndarray, Wo: np.ndarray,
                   global_layer: bool, n_heads: int = N_HEADS, n_kv: int = N_KV_HEADS, head_dim: int = HEAD_DIM,
                   rot_dim: int = ROTARY_DIM, window: int = WINDOW, base: float = ROPE_BASE) -> dict:
    """The attention half of one layer over a whole sequence, positions 0..P-1.

    x_bits: bf16 bit patterns [P][H]; Wq [nh*hd][H], Wk, Wv [nkv*hd][H],
    Wo [H][nh*hd]: dense float64 weights (dequantized ternary). Returns
    float64 q, k (after rotary on sliding layers), v, the attention output
    attn [P][nh*hd] and o = attn Wo^T [P][H]."""
    x = bf16_to_f64(x_bits)
    P = x.shape[0]
    q = (x @ Wq.T).reshape(P, n_heads, head_dim).transpose(1, 0, 2)  # [nh][P][hd]
    k = (x @ Wk.T).reshape(P, n_kv, head_dim).transpose(1, 0, 2)
    v = (x @ Wv.T).reshape(P, n_kv, head_dim).transpose(1, 0, 2)
    pos = np.arange(P)
    if not global_layer:
        q = rope(q, pos, rot_dim, base)
        k = rope(k, pos, rot_dim, base)
    win = 0 if global_layer else window
    pp, jj = np.meshgrid(pos, pos, indexing="ij")
    mask = (jj <= pp) & ((win == 0) | (pp - jj < win))  # visible(p, j, win) for every pair
    group = n_heads // n_kv
    attn = np.zeros((P, n_heads, head_dim))
    for h in range(n_heads):
        g = h // group
        s = (q[h] @ k[g].T) / np.sqrt(head_dim)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        attn[:, h, :] = p @ v[g]
    attn = attn.reshape(P, n_heads * head_dim)
    return dict(q=q, k=k, v=v, attn=attn, o=attn @ Wo.T)
