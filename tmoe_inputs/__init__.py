"""Seeded synthetic inputs for the ternary MoE expert layer.

This module only draws numbers. It holds none of the layer's arithmetic
(no ternarization, packing, routing or expert math). The CPU oracle and the
GPU library both consume what it produces; the GPU library additionally has
its own device implementation of the same counter-based generator (see
``ih12_normal``) so that multi-gigabyte weight sets can be drawn in HBM.

Workload shapes follow the Maple-Preview model card as reported on the
pages: hidden size 2048, 256 experts, top-8 routing, moe_intermediate_size
512, 24 layers (jj-blog, architecture section; ai.thesatyajit.com,
"The architecture around the quantization").

Weight generator (both sides implement it from its published definition):

* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
  easy as 1, 2, 3", SC'11). Element ``i`` of stream ``S`` uses the block
  cipher on counter ``(i, S, 0, 0)`` with key ``(KEY, 0)``. On the host this
  is NumPy's own ``numpy.random.Philox`` (which pre-increments its counter).
* Irwin-Hall(12) transform: the first three 64-bit output words are split
  into twelve little-endian 16-bit uniforms ``u_m`` and
  ``w = (sum(u_m) - 393210) * 2**-16``. The sum is an integer, so ``w`` is
  exactly representable in fp32 and identical on every implementation. Its
  variance is ``(2**32 - 1) / 2**32`` (unit to 1e-10), its support
  ``(-6, 6)``; it stands in for the N(0, 1) draws of the weight recipe.
* Router weights are ``fp32(0.02) * w`` (one IEEE fp32 multiply), i.e.
  N(0, 0.02) in the same Irwin-Hall approximation.

Activations (host only) are NumPy PCG64 normals rounded to bf16 (round to
nearest even); routing biases are NumPy PCG64 draws (Zipf / uniform).
"""
from __future__ import annotations

import numpy as np

KEY = 0x7E4A
HIDDEN = 2048
INTER = 512
N_EXPERTS = 256
TOP_K = 8
N_LAYERS = 24

MAT_GATE, MAT_UP, MAT_DOWN, MAT_ROUTER = 0, 1, 2, 3
MAT_ATTN_QKV, MAT_ATTN_O = 4, 5
ATTN_STD = np.float32(0.02)
ATTN_QKV_ROWS = 16 * 128 + 2 * 4 * 128  # query heads, then key and value heads (head_dim 128)
MAT_LMHEAD = 6
VOCAB = 151936
LMHEAD_STD = np.float32(0.02)
IH12_OFFSET = 393210  # 12 * (2**16 - 1) / 2
ROUTER_STD = np.float32(0.02)

# The five workloads: (name, tokens, bias kind, layers)
CONFIGS = {
    1: dict(name="ternary_linear_2048x512_T4", tokens=4, bias=None, layers=1),
    2: dict(name="moe_layer_decode_T1", tokens=1, bias=None, layers=1),
    3: dict(name="moe_layer_decode_T64_zipf1.1", tokens=64, bias="zipf", layers=1),
    4: dict(name="moe_layer_prefill_T4096_uniform", tokens=4096, bias="uniform", layers=1),
    5: dict(name="moe_stack24_T256_residual", tokens=256, bias=None, layers=24),
}


def stream_id(cfg: int, layer: int, expert: int, mat: int) -> int:
    """Unique Philox stream number (>= 1) for one weight matrix."""
    if not (0 <= cfg < 64 and 0 <= layer < 64 and 0 <= expert < 1024 and 0 <= mat < 8):
        raise ValueError("stream coordinates out of range")
    return 1 + (((cfg * 64 + layer) * 1024 + expert) * 8 + mat)


def philox_words(stream: int, first: int, n: int) -> np.ndarray:
    """[n, 4] uint64 Philox4x64-10 blocks for counters (first..first+n-1, stream, 0, 0)."""
    if stream < 1:
        raise ValueError("stream must be >= 1")
    g = np.random.Philox(key=KEY, counter=(stream << 64) + first - 1)
    return g.random_raw(4 * n).reshape(n, 4)


def ih12_normal(stream: int, n: int, first: int = 0) -> np.ndarray:
    """n float32 Irwin-Hall(12) draws of one stream (see module docstring)."""
    words = philox_words(stream, first, n)[:, :3].copy()
    s = words.view(np.uint16).reshape(n, 12).sum(axis=1, dtype=np.int32) - IH12_OFFSET
    return (s.astype(np.float32) * np.float32(2.0 ** -16)).astype(np.float32)


def expert_matrix(cfg: int, layer: int, expert: int, mat: int) -> np.ndarray:
    """Raw fp32 weights of one expert matrix, [out][in] (F.linear orientation)."""
    shape = (INTER, HIDDEN) if mat in (MAT_GATE, MAT_UP) else (HIDDEN, INTER)
    w = ih12_normal(stream_id(cfg, layer, expert, mat), shape[0] * shape[1])
    return w.reshape(shape)


def linear_matrix(cfg: int = 1, rows: int = INTER, cols: int = HIDDEN) -> np.ndarray:
    """Raw fp32 weights for the single ternary linear workload."""
    return ih12_normal(stream_id(cfg, 0, 0, MAT_GATE), rows * cols).reshape(rows, cols)


def router_matrix(cfg: int, layer: int, experts: int = N_EXPERTS, hidden: int = HIDDEN) -> np.ndarray:
    """fp32 router weights [E][H], fp32(0.02) * Irwin-Hall(12)."""
    w = ih12_normal(stream_id(cfg, layer, 1023, MAT_ROUTER), experts * hidden)
    return (w * ROUTER_STD).astype(np.float32).reshape(experts, hidden)


def attn_qkv_matrix(cfg: int, layer: int, rows: int = ATTN_QKV_ROWS, hidden: int = HIDDEN) -> np.ndarray:
    """Raw fp32 [q; k; v] projection rows [rows][hidden]: fp32(0.02) * Irwin-Hall(12)."""
    w = ih12_normal(stream_id(cfg, layer, 0, MAT_ATTN_QKV), rows * hidden)
    return (w * ATTN_STD).astype(np.float32).reshape(rows, hidden)


def attn_o_matrix(cfg: int, layer: int, hidden: int = HIDDEN, width: int = HIDDEN) -> np.ndarray:
    """Raw fp32 output projection [hidden][width]: fp32(0.02) * Irwin-Hall(12)."""
    w = ih12_normal(stream_id(cfg, layer, 0, MAT_ATTN_O), hidden * width)
    return (w * ATTN_STD).astype(np.float32).reshape(hidden, width)


def lm_head_rows(cfg: int, v0: int, v1: int, hidden: int = HIDDEN) -> np.ndarray:
    """Rows v0..v1-1 of the bf16 output embedding, as uint16 bit patterns
    [v1 - v0][hidden]: bf16 (nearest even) of fp32(0.02) * Irwin-Hall(12),
    element v * hidden + i drawn from counter v * hidden + i of one stream."""
    w = ih12_normal(stream_id(cfg, 0, 0, MAT_LMHEAD), (v1 - v0) * hidden, first=v0 * hidden)
    return f32_to_bf16_bits((w * LMHEAD_STD).astype(np.float32)).reshape(v1 - v0, hidden)


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([KEY, *words])))


def router_bias(cfg: int, kind: str | None, experts: int = N_EXPERTS) -> np.ndarray | None:
    """Synthetic routing skew added to the router logits.

    zipf: b_e = -1.1 * ln(rank_e), rank a seeded permutation of 1..E (the log of an
          unnormalised Zipf(s=1.1) law), so a few experts attract most tokens.
    uniform: b_e ~ U(-0.1, 0.1).
    """
    if kind is None:
        return None
    g = _rng(cfg, 4)
    if kind == "zipf":
        rank = g.permutation(experts) + 1
        return (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    if kind == "uniform":
        return g.uniform(-0.1, 0.1, size=experts).astype(np.float32)
    raise ValueError(kind)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(cfg: int, tokens: int, hidden: int = HIDDEN, layer: int = 0) -> np.ndarray:
    """bf16 activations N(0, 1) as uint16 bit patterns [T][H]."""
    g = _rng(cfg, layer, 5)
    x = g.standard_normal((tokens, hidden), dtype=np.float32)
    return f32_to_bf16_bits(x)


def integer_activations(seed: int, tokens: int, hidden: int, lim: int = 8) -> np.ndarray:
    """bf16 bit patterns of small integers in [-lim, lim] (exact-sum test inputs)."""
    g = _rng(seed, 6)
    x = g.integers(-lim, lim + 1, size=(tokens, hidden)).astype(np.float32)
    return f32_to_bf16_bits(x)
