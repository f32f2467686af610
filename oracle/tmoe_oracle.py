"""CPU oracle for the ternary Mixture-of-Experts expert layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never uses it and shares no code with it.

It computes, plainly and slowly, in NumPy float64 without blocking or fusion,
what the layer is defined to compute. Sources (the pages are the authority):

* ai.thesatyajit.com, "Maple-Preview: a 20B reasoning model where 97% of the
  weights are -1, 0, or +1":
  - "The claim, verified from the bytes": every weight row holds exactly the
    three values {-s, 0, +s} with one scale per output channel (the BitNet
    b1.58 shape); absmean ternarization is named.
  - "The 5.31 GB claim reconciles": five trits packed into one byte
    (3**5 = 243 <= 256); log2(3) bits per trit is the floor.
  - "The claim, verified from the bytes" (router paragraph): the MoE router
    stays full precision and chooses 8 of 256 experts from its logits.
  - "The shipped code does no quantization": an expert maps x to
    o = Wd h with h = SiLU(min(g, 7)) * clip(u, -7, 7), g = Wg x, u = Wu x.
* codeinsider.com.br, "Pesos ternarios": a ternary weight skips (0), adds
  (+1) or subtracts (-1) the activation; "256 experts, 8 ativos": 8 of 256
  experts are active per token.
* jj-blog (Maple-Preview news), architecture list: hidden 2048, 256 experts,
  8 per token, no shared expert, moe_intermediate_size 512, 24 layers.

Readings where the pages are silent:
scale = fp32 of the fp64 mean of |W_row| summed in index order; trit =
sign(W) where 2|W| > s, else 0 (RoundClip(W/s) with ties to zero, no
epsilon); digit d = t + 1, little-endian base 3 along the input dimension,
padding trits 0; router weights fp32 [E][H] (F.linear orientation) plus an
optional bias; top-k by descending logit with ties to the lower expert index;
softmax over the k selected logits; SiLU activation; clamp c = 7; expert
intermediates kept in float64; combine = routing-weighted sum; residual =
bf16(fp32(x) + y).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

_POW3 = np.array([1, 3, 9, 27, 81], dtype=np.int64)


# ----------------------------------------------------------------------------
# bf16 / fp32 conversions (input format and residual rounding)
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """bf16 nearest-even rounding of finite fp32 values, returned as uint16 bits.

    Written from the rounding rule: keep the top 16 bits, add one unit of the
    kept part when the dropped half-word is above one half, or exactly one
    half with an odd kept part.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    keep = u >> 16
    drop = u & 0xFFFF
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.int64)).astype(np.uint16)


# ----------------------------------------------------------------------------
# O1 ternarization (absmean, per output row)
# ----------------------------------------------------------------------------
def ternarize_absmean(W: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Absmean ternarization of fp32 W [R][K] -> (trits int8 [R][K], scale fp32 [R]).

    ai.thesatyajit.com, "The claim, verified from the bytes": rows are
    {-s, 0, +s} with a per-output-channel scale, as absmean ternarization
    produces. s_r = mean_i |W_ri| (fp64, index order, one rounding to fp32);
    t_ri = RoundClip(W_ri / s_r, -1, 1) = sign(W_ri) if 2|W_ri| > s_r else 0.
    An all-zero row gives s = 0 and all-zero trits.
    """
    W = np.asarray(W, dtype=np.float32)
    R, K = W.shape
    a = np.abs(W.astype(np.float64))
    s = (np.cumsum(a, axis=1)[:, -1] / K).astype(np.float32) if K else np.zeros(R, np.float32)
    keep = 2.0 * a > s.astype(np.float64)[:, None]
    t = np.where(keep, np.sign(W.astype(np.float64)), 0.0).astype(np.int8)
    return t, s


def dequantize(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Dense float64 weights s_r * t_ri."""
    return t.astype(np.float64) * np.asarray(s, dtype=np.float64)[:, None]


# ----------------------------------------------------------------------------
# O2/O3 five-trits-per-byte packing
# ----------------------------------------------------------------------------
def packed_row_bytes(K: int) -> int:
    """ceil(K / 5) bytes per row."""
    return -(-K // 5)


def pack_trits(t: np.ndarray, ldp: int | None = None) -> np.ndarray:
    """Trits int8 [R][K] in {-1,0,1} -> bytes uint8 [R][ldp].

    ai.thesatyajit.com, "The 5.31 GB claim reconciles": five trits per byte,
    3**5 = 243 <= 256. Digit d = t + 1; byte j of a row is
    sum_q d_{5j+q} * 3**q; trits past K are 0 (digit 1). Bytes [ceil(K/5), ldp)
    are zero in the returned array (not part of the format).
    """
    t = np.asarray(t, dtype=np.int8)
    R, K = t.shape
    Kb = packed_row_bytes(K)
    ldp = Kb if ldp is None else ldp
    if ldp < Kb:
        raise ValueError("ldp < ceil(K/5)")
    if np.any((t < -1) | (t > 1)):
        raise ValueError("trits must be in {-1, 0, 1}")
    d = np.ones((R, Kb * 5), dtype=np.int64)
    d[:, :K] = t.astype(np.int64) + 1
    b = (d.reshape(R, Kb, 5) * _POW3).sum(axis=2)
    out = np.zeros((R, ldp), dtype=np.uint8)
    out[:, :Kb] = b.astype(np.uint8)
    return out


def unpack_trits(P: np.ndarray, K: int) -> np.ndarray:
    """Bytes uint8 [R][>=ceil(K/5)] -> trits int8 [R][K]: t = ((b div 3**q) mod 3) - 1."""
    P = np.asarray(P, dtype=np.uint8)
    Kb = packed_row_bytes(K)
    b = P[:, :Kb].astype(np.int64)
    if np.any(b > 242):
        raise ValueError("packed byte > 242 is not a valid 5-trit code")
    d = (b[:, :, None] // _POW3) % 3
    return (d.reshape(P.shape[0], Kb * 5)[:, :K] - 1).astype(np.int8)


# ----------------------------------------------------------------------------
# O4 ternary linear
# ----------------------------------------------------------------------------
def ternary_linear(t: np.ndarray, s: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[n][o] = s_o * sum_i t_oi x_ni, float64 (x given as float64 values).

    codeinsider.com.br, "Pesos ternarios": t = 0 skips, +1 adds, -1 subtracts;
    the result equals the dense product with the dequantized matrix.
    """
    return (np.asarray(x, dtype=np.float64) @ t.astype(np.float64).T) * np.asarray(s, np.float64)[None, :]


# ----------------------------------------------------------------------------
# O5 router: full-precision logits, top-k, softmax over the k selected
# ----------------------------------------------------------------------------
def _exact_logit(x_row: np.ndarray, w_row: np.ndarray, b: float | None) -> Fraction:
    acc = Fraction(0)
    for xi, wi in zip(x_row.tolist(), w_row.tolist()):
        if xi != 0.0 and wi != 0.0:
            acc += Fraction(xi) * Fraction(wi)
    if b is not None:
        acc += Fraction(b)
    return acc


def router_topk(x: np.ndarray, Wr: np.ndarray, bias: np.ndarray | None, k: int):
    """Router of one MoE layer.

    ai.thesatyajit.com, "The claim, verified from the bytes": the router is
    kept in full precision and picks 8 of 256 experts by the margins between
    logits. Logits l[t][e] = sum_i x[t][i] * Wr[e][i] (+ bias[e]); the k
    largest in descending order, equal logits to the lower index; weights
    softmax over the k selected logits.

    The ranking is that of the exact logits: float64 values decide unless two
    candidates lie within the float64 error bound of each other, in which case
    those candidates are recomputed exactly as rationals.

    Returns (idx int32 [T][k], w float64 [T][k], logits float64 [T][E],
    n_exact = number of tokens that needed the exact recomputation).
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(Wr, dtype=np.float32).astype(np.float64)
    T, H = x.shape
    E = W.shape[0]
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    b = None if bias is None else np.asarray(bias, dtype=np.float32).astype(np.float64)
    L = x @ W.T
    A = np.abs(x) @ np.abs(W).T
    if b is not None:
        L = L + b[None, :]
        A = A + np.abs(b)[None, :]
    u = 2.0 ** -53
    n = H + 2
    err = 2.0 * (n * u / (1.0 - n * u)) * A  # generous bound on |L - exact|
    idx = np.zeros((T, k), dtype=np.int32)
    wts = np.zeros((T, k), dtype=np.float64)
    n_exact = 0
    experts = np.arange(E)
    for t in range(T):
        order = np.lexsort((experts, -L[t]))
        m = min(k + 1, E)
        top = order[:m]
        ambiguous = False
        for a_, b_ in zip(top[:-1], top[1:]):
            if L[t, a_] - L[t, b_] <= err[t, a_] + err[t, b_]:
                ambiguous = True
                break
        if ambiguous:
            n_exact += 1
            # every expert whose interval reaches the m-th largest lower edge is a candidate
            floor = L[t, top[-1]] - err[t, top[-1]]
            cand = [e for e in range(E) if L[t, e] + err[t, e] >= floor]
            ex = {e: _exact_logit(x[t], W[e], None if b is None else b[e]) for e in cand}
            cand.sort(key=lambda e: (-ex[e], e))
            order = np.array(cand + [e for e in order if e not in ex], dtype=np.int64)
        sel = order[:k]
        idx[t] = sel
        ls = L[t, sel]
        p = np.exp(ls - ls.max())
        wts[t] = p / p.sum()
    return idx, wts, L, n_exact


# ----------------------------------------------------------------------------
# LM head: untied bf16 output embedding, logits over the vocabulary, top-k
# ----------------------------------------------------------------------------
def lm_head_topk(x_bits: np.ndarray, W_bits: np.ndarray, k: int, chunk: int = 16384):
    """Output head of the model and the k most likely next tokens.

    ai.thesatyajit.com, "The 5.31 GB claim reconciles, and the leftover is the
    vocabulary": the input and output embedding tables (151,936 tokens x 2048)
    are untied and stay un-quantized; at the model's compression they are
    about a quarter of the file. Readings: the output table is bf16 [V][H]
    (two bytes per entry, which is what the page's file-size arithmetic
    implies), the head's input is the final hidden state in bf16 (the final
    norm is outside this step), logits l[t][v] = sum_i x[t][i] * W[v][i], and
    the k largest logits are returned in descending order with equal logits to
    the lower token id (the router's reading).

    float64 decides unless two candidates lie within the float64 error bound,
    in which case they are recomputed exactly as rationals (as in router_topk).
    W_bits may be any array-like of uint16 rows (it is read `chunk` rows at a
    time). Returns (idx int32 [T][k], val float64 [T][k], logits float64
    [T][V], n_exact).
    """
    x = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16))
    T, H = x.shape
    V = W_bits.shape[0]
    if not (1 <= k <= V):
        raise ValueError("need 1 <= k <= V")
    L = np.empty((T, V))
    A = np.empty((T, V))
    for v0 in range(0, V, chunk):
        Wc = bf16_to_f64(np.asarray(W_bits[v0:v0 + chunk], dtype=np.uint16))
        L[:, v0:v0 + Wc.shape[0]] = x @ Wc.T
        A[:, v0:v0 + Wc.shape[0]] = np.abs(x) @ np.abs(Wc).T
    u = 2.0 ** -53
    n = H + 2
    err = 2.0 * (n * u / (1.0 - n * u)) * A
    idx = np.zeros((T, k), dtype=np.int32)
    val = np.zeros((T, k))
    n_exact = 0
    ids = np.arange(V)
    for t in range(T):
        order = np.lexsort((ids, -L[t]))
        m = min(k + 1, V)
        top = order[:m]
        ambiguous = any(L[t, a_] - L[t, b_] <= err[t, a_] + err[t, b_] for a_, b_ in zip(top[:-1], top[1:]))
        if ambiguous:
            n_exact += 1
            floor = L[t, top[-1]] - err[t, top[-1]]
            cand = [int(v) for v in np.nonzero(L[t] + err[t] >= floor)[0]]
            ex = {v: _exact_logit(x[t], bf16_to_f64(np.asarray(W_bits[v], dtype=np.uint16)), None) for v in cand}
            cand.sort(key=lambda v: (-ex[v], v))
            rest = [int(v) for v in order[: m + len(cand)] if int(v) not in ex]
            order = np.array(cand + rest, dtype=np.int64)
        idx[t] = order[:k]
        val[t] = L[t, order[:k]]
    return idx, val, L, n_exact


# ----------------------------------------------------------------------------
# O6 token -> expert grouping
# ----------------------------------------------------------------------------
def group_by_expert(idx: np.ndarray, E: int):
    """Stable grouping of the T*k (token, slot) pairs by expert.

    Entries are ordered by expert, then by token (a token selects an expert at
    most once). Returns counts [E], offsets [E+1], sorted_token [T*k],
    sorted_slot [T*k] and pos [T*k] (pos[t*k + j] = grouped position of the
    pair (t, j)).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    entries = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    counts = np.zeros(E, dtype=np.int32)
    for e, _, _ in entries:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_token = np.array([t for _, t, _ in entries], dtype=np.int32).reshape(-1)
    sorted_slot = np.array([j for _, _, j in entries], dtype=np.int32).reshape(-1)
    pos = np.zeros(T * k, dtype=np.int32)
    for p, (_, t, j) in enumerate(entries):
        pos[t * k + j] = p
    return counts, offsets, sorted_token, sorted_slot, pos


# ----------------------------------------------------------------------------
# O7 expert FFN, O8 combine, O9 residual
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    # for z below about -709, e^(-z) is +inf in fp64 and z / inf = -0, the limit
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, gate: np.ndarray, up: np.ndarray, down: np.ndarray, clamp: float = 7.0):
    """One expert on float64 rows x [n][H] with dense float64 weights.

    The expert forward of ai.thesatyajit.com, "The shipped code does no
    quantization": with g = Wg x and u = Wu x (weights in [out][in] order),
    h = SiLU(min(g, c)) * min(max(u, -c), c) elementwise and o = Wd h; the
    activation is SiLU and c = 7 (c = inf leaves g and u unclamped).
    Returns (g, u, h, o), all float64.
    """
    g = x @ gate.T
    u = x @ up.T
    h = silu(np.minimum(g, clamp)) * np.clip(u, -clamp, clamp)
    o = h @ down.T
    return g, u, h, o


def moe_layer(x_bits: np.ndarray, Wr: np.ndarray, bias, get_expert, k: int = 8, clamp: float = 7.0):
    """The whole layer on bf16 input rows.

    get_expert(e) -> (gate_fp32 [I][H], up_fp32 [I][H], down_fp32 [H][I]) raw
    weights; they are ternarized here (O1) and used dequantized.

    Returns a dict with idx, w, logits, grouping, G/U/H/O in grouped order
    (row p of each is the pair with grouped position p) and Y fp64 [T][H]
    (round to fp32 for the layer output).
    """
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    E = np.asarray(Wr).shape[0]
    idx, w, L, n_exact = router_topk(x, Wr, bias, k)
    counts, offsets, sorted_token, sorted_slot, pos = group_by_expert(idx, E)
    I = None
    G = U = Hh = O = None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Wg, Wu, Wd = get_expert(e)
        tg, sg = ternarize_absmean(Wg)
        tu, su = ternarize_absmean(Wu)
        td, sd = ternarize_absmean(Wd)
        toks = sorted_token[lo:hi]
        g, u, h, o = expert_ffn(x[toks], dequantize(tg, sg), dequantize(tu, su), dequantize(td, sd), clamp)
        if G is None:
            I = g.shape[1]
            G = np.zeros((T * k, I)); U = np.zeros((T * k, I)); Hh = np.zeros((T * k, I))
            O = np.zeros((T * k, H))
        G[lo:hi], U[lo:hi], Hh[lo:hi], O[lo:hi] = g, u, h, o
    Y = combine(O, w, pos)
    return dict(idx=idx, w=w, logits=L, n_exact=n_exact, counts=counts, offsets=offsets,
                sorted_token=sorted_token, sorted_slot=sorted_slot, pos=pos,
                G=G, U=U, H=Hh, O=O, Y=Y)


def combine(O: np.ndarray, w: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Y[t] = sum_j w[t][j] * O[pos[t*k + j]] in float64 (slot order)."""
    T, k = w.shape
    Y = np.zeros((T, O.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            Y[t] += np.float64(w[t, j]) * O[pos[t * k + j]]
    return Y


def residual_bf16(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """x_next = bf16_RNE(fp32(x) + fp32(y)) (one fp32 add, then one bf16 rounding)."""
    xf = bf16_to_f64(x_bits).astype(np.float32)
    s = (xf + np.asarray(y, dtype=np.float32)).astype(np.float32)
    return f32_to_bf16_rne(s)


def max_normalized_error(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got_r - ref_r||_inf / ||ref_r||_inf (rows with ref = 0 use 1)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())
