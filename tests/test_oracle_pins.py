"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself (hand-worked examples, closed forms, exhaustive enumeration,
library routines, brute force). CPU only."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import tmoe_inputs as ti

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def _figs():
    """Page figures by name: numbers as float, lists of numbers as int lists."""
    out = {}
    for name, value, _ in _read_golden("page_figures.txt"):
        out[name] = [int(v) for v in value.split()] if " " in value else float(value)
    return out


# ---------------------------------------------------------------- packing (O2/O3)
def test_pack_hand_examples():
    for trits, expect in _read_golden("pack_examples.txt"):
        t = np.array([[int(v) for v in trits.split(",")]], dtype=np.int8)
        want = [int(v) for v in expect.split(",")]
        got = O.pack_trits(t)[0].tolist()
        assert got == want, (trits, got, want)
        assert O.unpack_trits(np.array([want], np.uint8), t.shape[1]).tolist() == t.tolist()


def test_pack_exhaustive_bijection():
    # every one of the 3^5 = 243 trit 5-tuples maps to a distinct byte in 0..242
    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=5)), dtype=np.int8)
    codes = O.pack_trits(tuples)[:, 0].astype(int)
    assert sorted(codes.tolist()) == list(range(243))
    back = O.unpack_trits(codes.astype(np.uint8)[:, None], 5)
    assert np.array_equal(back, tuples)
    # negating every trit mirrors the code: code(-t) = 242 - code(t)
    neg = O.pack_trits(-tuples)[:, 0].astype(int)
    assert np.array_equal(neg, 242 - codes)
    # first trit is the least significant base-3 digit
    for q in range(5):
        e = np.zeros((1, 5), np.int8)
        e[0, q] = 1
        assert int(O.pack_trits(e)[0, 0]) == 121 + 3 ** q


@pytest.mark.parametrize("K", list(range(1, 18)) + [512, 2048])
def test_pack_roundtrip_random(K):
    g = np.random.default_rng(K)
    t = g.integers(-1, 2, size=(7, K)).astype(np.int8)
    P = O.pack_trits(t, ldp=-(-K // 5) + 3)
    assert P.shape == (7, -(-K // 5) + 3)
    assert P.max() <= 242
    assert np.array_equal(O.unpack_trits(P, K), t)
    # padding trits past K are zero (digit 1)
    Kb = -(-K // 5)
    full = O.unpack_trits(P, Kb * 5)
    assert np.all(full[:, K:] == 0)


def test_unpack_rejects_invalid_bytes():
    with pytest.raises(ValueError):
        O.unpack_trits(np.array([[243]], np.uint8), 5)


def test_packed_sizes_closed_form():
    figs = _figs()
    assert 3 ** int(figs["trits_per_byte"]) == int(figs["codes_per_byte"]) <= 256
    assert abs(math.log2(3) - figs["entropy_floor_bits"]) < 5e-4
    H, I, E, L = int(figs["hidden"]), int(figs["moe_intermediate"]), int(figs["n_experts"]), int(figs["n_layers"])
    assert O.packed_row_bytes(H) == 410 and O.packed_row_bytes(I) == 103
    per_expert = 2 * I * O.packed_row_bytes(H) + H * O.packed_row_bytes(I) + 4 * (2 * I + H)
    assert per_expert == 643072
    assert per_expert * E * L == 3951034368
    trits = 3 * I * H * E * L
    bits_with_scales = 8 * per_expert * E * L / trits
    # five trits per byte is 1.6 bits; fp32 row scales bring it to 1.635, just
    # under the page's 1.65 and above the log2(3) floor
    assert abs(bits_with_scales - 1.635) < 1e-3
    assert figs["entropy_floor_bits"] < bits_with_scales < figs["bits_per_ternary_weight"]
    # the page's own census: (5.31 GB - 2 bytes x 0.64B full-precision) / 19.58B trits
    page_bits = 8 * (figs["packed_checkpoint_bytes"] - 2 * figs["full_precision_params"]) / figs["ternary_params"]
    assert abs(page_bits - figs["bits_per_ternary_weight"]) < 0.01


# ---------------------------------------------------------------- ternarization (O1)
def test_ternarize_hand_examples():
    for w, t, s in _read_golden("ternarize_examples.txt"):
        W = np.array([[float(v) for v in w.split(",")]], np.float32)
        tt, ss = O.ternarize_absmean(W)
        assert tt[0].tolist() == [int(v) for v in t.split(",")]
        assert ss[0] == np.float32(float(s))


def test_ternarize_roundclip_library():
    # equals RoundClip(W/s, -1, 1) with numpy's round-half-to-even, computed in float64
    g = np.random.default_rng(1)
    W = g.standard_normal((64, 300)).astype(np.float32)
    t, s = O.ternarize_absmean(W)
    ref = np.clip(np.round(W.astype(np.float64) / s.astype(np.float64)[:, None]), -1, 1)
    assert np.array_equal(t, ref.astype(np.int8))
    # scale is the exact mean of |W| rounded once to fp32 (exact-rational check on a few rows)
    for r in range(4):
        exact = sum(Fraction(float(abs(v))) for v in W[r]) / W.shape[1]
        assert s[r] == np.float32(float(exact))


def test_ternarize_three_symmetric_values_per_row():
    W = ti.expert_matrix(2, 0, 0, ti.MAT_GATE)[:128]
    t, s = O.ternarize_absmean(W)
    D = O.dequantize(t, s)
    for r in range(D.shape[0]):
        vals = set(np.unique(D[r]).tolist())
        assert vals == {-float(s[r]), 0.0, float(s[r])}
        assert s[r] > 0


def test_ternarize_special_rows():
    W = np.array([[0.3] * 9, [-2.5] * 9, [0.0] * 9], np.float32)
    t, s = O.ternarize_absmean(W)
    assert s[0] == np.float32(0.3) and np.all(t[0] == 1)
    assert s[1] == np.float32(2.5) and np.all(t[1] == -1)
    assert s[2] == 0 and np.all(t[2] == 0)


def _phi(z):
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def test_zero_fraction_gaussian_closed_form():
    # For N(0, sigma^2), E|W| = sigma*sqrt(2/pi); the zero band |W| <= s/2 has mass
    # 2*Phi(1/sqrt(2*pi)) - 1 = 0.31006. The page's 38-43% (ai.thesatyajit.com,
    # "The claim, verified from the bytes") is not what a Gaussian row gives.
    p = 2 * _phi(1 / math.sqrt(2 * math.pi)) - 1
    assert abs(p - 0.31006) < 1e-5
    g = np.random.default_rng(2)
    W = g.standard_normal((512, 2048)).astype(np.float32)
    t, s = O.ternarize_absmean(W)
    z = (t == 0).mean(axis=1)
    se = math.sqrt(p * (1 - p) / 2048)
    assert abs(z.mean() - p) < 4 * se / math.sqrt(512)
    assert np.all(np.abs(z - p) < 6 * se)
    assert abs(s.mean() - math.sqrt(2 / math.pi)) < 2e-3


def test_zero_fraction_heavy_tail_reproduces_page_band():
    # Laplace(b): E|W| = b and P(|W| <= b/2) = 1 - exp(-1/2) = 0.39347, inside the
    # page's 38-43% band for trained rows.
    figs = _figs()
    p = 1 - math.exp(-0.5)
    assert figs["zero_fraction_low"] < p < figs["zero_fraction_high"]
    g = np.random.default_rng(3)
    W = g.laplace(size=(256, 2048)).astype(np.float32)
    z = (O.ternarize_absmean(W)[0] == 0).mean(axis=1)
    se = math.sqrt(p * (1 - p) / 2048)
    assert abs(z.mean() - p) < 4 * se / math.sqrt(256)
    assert np.all((z > p - 6 * se) & (z < p + 6 * se))


# ---------------------------------------------------------------- ternary linear (O4)
def _add_skip_subtract(t, s, x):
    # codeinsider.com.br, "Pesos ternarios": weight 0 skips, +1 adds, -1 subtracts
    y = []
    for o in range(len(t)):
        acc = 0
        for i in range(len(t[o])):
            if t[o][i] == 0:
                continue
            elif t[o][i] == 1:
                acc = acc + x[i]
            else:
                acc = acc - x[i]
        y.append(s[o] * acc)
    return y


@pytest.mark.parametrize("R,K", [(1, 1), (3, 7), (9, 23), (5, 11), (2, 16)])
def test_ternary_linear_brute_force(R, K):
    g = np.random.default_rng(R * 100 + K)
    t = g.integers(-1, 2, size=(R, K)).astype(np.int8)
    s = (2.0 ** g.integers(-3, 4, size=R)).astype(np.float32)
    x = g.integers(-8, 9, size=(3, K)).astype(np.float64)
    y = O.ternary_linear(t, s, x)
    for n in range(3):
        brute = _add_skip_subtract(t.tolist(), [Fraction(float(v)) for v in s], [Fraction(int(v)) for v in x[n]])
        assert [Fraction(v) for v in y[n].tolist()] == brute


def test_ternary_linear_hand_example():
    t = np.array([[1, 0, -1], [0, 1, 1]], np.int8)
    y = O.ternary_linear(t, np.array([0.5, 2.0], np.float32), np.array([[3.0, -1.0, 2.0]]))
    assert y.tolist() == [[0.5, 2.0]]


def test_ternary_linear_torch_library():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(4)
    t = g.integers(-1, 2, size=(37, 61)).astype(np.int8)
    s = g.random(37).astype(np.float32)
    x = g.standard_normal((5, 61))
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(O.dequantize(t, s))).numpy()
    assert np.allclose(O.ternary_linear(t, s, x), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- router (O5)
def test_router_matches_library_sort_and_softmax():
    scipy_special = pytest.importorskip("scipy.special")
    g = np.random.default_rng(5)
    x = O.bf16_to_f64(ti.f32_to_bf16_bits(g.standard_normal((16, 64)).astype(np.float32)))
    Wr = (g.standard_normal((32, 64)) * 0.02).astype(np.float32)
    b = g.uniform(-0.1, 0.1, 32).astype(np.float32)
    idx, w, L, n_exact = O.router_topk(x, Wr, b, 8)
    Lref = x @ Wr.astype(np.float64).T + b.astype(np.float64)
    for t in range(16):
        assert idx[t].tolist() == np.argsort(-Lref[t], kind="stable")[:8].tolist()
        assert abs(w[t].sum() - 1) < 1e-14
        assert np.allclose(w[t], scipy_special.softmax(Lref[t][idx[t]]), rtol=1e-13)
    # k = E is a full softmax; k = 1 gives weight 1
    idxE, wE, _, _ = O.router_topk(x, Wr, b, 32)
    for t in range(16):
        assert np.allclose(wE[t][np.argsort(idxE[t])], scipy_special.softmax(Lref[t]), rtol=1e-12)
    _, w1, _, _ = O.router_topk(x, Wr, b, 1)
    assert np.all(w1 == 1.0)


def test_router_ties_go_to_lower_index():
    g = np.random.default_rng(6)
    x = O.bf16_to_f64(ti.f32_to_bf16_bits(g.standard_normal((4, 32)).astype(np.float32)))
    Wr = (g.standard_normal((16, 32)) * 0.02).astype(np.float32)
    Wr[11] = Wr[3]  # equal logits for experts 3 and 11
    Wr[12] = Wr[3]
    big = np.zeros(16, np.float32)
    big[[3, 11, 12]] = 10.0
    idx, _, _, n_exact = O.router_topk(x, Wr, big, 4)
    assert n_exact == 4
    for t in range(4):
        assert idx[t][:3].tolist() == [3, 11, 12]


def test_router_exact_path_resolves_float64_collision():
    # logits 1 and 1 + 2^-60 collide in float64; the exact ranking puts expert 1 first
    x = np.zeros((1, 4))
    x[0, 0] = 1.0
    x[0, 1] = 2.0 ** -60
    Wr = np.zeros((3, 4), np.float32)
    Wr[0, 0] = 1.0
    Wr[1, 0] = 1.0
    Wr[1, 1] = 1.0
    Wr[2, 2] = 1.0
    idx, _, L, n_exact = O.router_topk(x, Wr, None, 2)
    assert L[0, 0] == L[0, 1]
    assert n_exact == 1
    assert idx[0].tolist() == [1, 0]


# ------------------------------------------------------------------ LM head
def test_lm_head_table_size_matches_page():
    figs = _figs()
    V, H = int(figs["vocab"]), int(figs["hidden"])
    table = V * H * 2  # one bf16 table
    assert table == 622329856
    # two untied tables plus the 24 full-precision routers are the page's
    # ~0.64B full-precision parameters at two bytes each (1.27 GB)
    routers = int(figs["n_layers"]) * int(figs["n_experts"]) * H
    assert abs(2 * V * H + routers - figs["full_precision_params"]) / figs["full_precision_params"] < 0.01
    assert abs(2 * (2 * V * H + routers) - figs["embedding_tables_bytes"]) / figs["embedding_tables_bytes"] < 0.01
    # "about a quarter of the entire file"
    assert 0.2 < 2 * table / figs["packed_checkpoint_bytes"] < 0.3


def _exact_sorted(xb, Wb):
    xf, Wf = O.bf16_to_f64(xb), O.bf16_to_f64(Wb)
    out = []
    for t in range(xf.shape[0]):
        ex = []
        for v in range(Wf.shape[0]):
            acc = Fraction(0)
            for a, b in zip(xf[t].tolist(), Wf[v].tolist()):
                acc += Fraction(a) * Fraction(b)
            ex.append(acc)
        out.append((ex, sorted(range(Wf.shape[0]), key=lambda v: (-ex[v], v))))
    return out


@pytest.mark.parametrize("V,H,k", [(23, 9, 5), (40, 33, 1), (17, 64, 17)])
def test_lm_head_brute_force(V, H, k):
    # exact rational logits by a plain double loop; the oracle's float64 logits
    # lie within its bound and its ranking is the exact one
    g = np.random.default_rng(V * 100 + H)
    xb = O.f32_to_bf16_rne(g.standard_normal((2, H)).astype(np.float32))
    Wb = O.f32_to_bf16_rne((g.standard_normal((V, H)) * 0.05).astype(np.float32))
    idx, val, L, _ = O.lm_head_topk(xb, Wb, k)
    for t, (ex, order) in enumerate(_exact_sorted(xb, Wb)):
        assert idx[t].tolist() == order[:k]
        for v in range(V):
            assert abs(L[t, v] - float(ex[v])) <= 1e-12 * (1.0 + abs(float(ex[v])))
        assert np.array_equal(val[t], L[t, idx[t]])


def test_lm_head_duplicate_rows_and_float64_collision():
    H = 4
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = 2.0 ** -60
    W = np.zeros((5, H), np.float32)
    W[1, 0] = 1.0            # logit 1
    W[3, 0] = 1.0            # logit 1 + 2^-60: collides with row 1 in float64
    W[3, 1] = 1.0
    W[4] = W[1]              # exact duplicate of row 1
    W[0, 2] = 1.0            # logit 0
    xb, Wb = O.f32_to_bf16_rne(x), O.f32_to_bf16_rne(W)
    idx, _, L, n_exact = O.lm_head_topk(xb, Wb, 3)
    assert L[0, 1] == L[0, 3] == L[0, 4]
    assert n_exact == 1
    assert idx[0].tolist() == [3, 1, 4]


def test_lm_head_k1_is_library_argmax():
    g = np.random.default_rng(5)
    xb = O.f32_to_bf16_rne(g.standard_normal((3, 128)).astype(np.float32))
    Wb = O.f32_to_bf16_rne((g.standard_normal((500, 128)) * 0.02).astype(np.float32))
    idx, _, L, _ = O.lm_head_topk(xb, Wb, 1)
    ref = O.bf16_to_f64(xb) @ O.bf16_to_f64(Wb).T
    assert np.array_equal(idx[:, 0], np.argmax(ref, axis=1))


# ---------------------------------------------------------------- grouping (O6)
def test_grouping_matches_stable_argsort():
    g = np.random.default_rng(7)
    T, k, E = 50, 8, 64
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, st, ss, pos = O.group_by_expert(idx, E)
    tok = np.repeat(np.arange(T), k)
    order = np.argsort(idx.ravel().astype(np.int64) * T + tok, kind="stable")
    assert np.array_equal(st, order // k) and np.array_equal(ss, order % k)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(idx.ravel()[order], np.repeat(np.arange(E), counts))
    inv = np.empty(T * k, np.int64)
    inv[order] = np.arange(T * k)
    assert np.array_equal(pos, inv)


# ---------------------------------------------------------------- expert FFN / combine (O7, O8, O9)
def test_expert_ffn_matches_torch_forward():
    # ai.thesatyajit.com, "The shipped code does no quantization": the expert
    # forward evaluated step by step with torch's float64 matmul, clamp and silu
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    g = np.random.default_rng(8)
    H, I = 40, 24
    Wg, Wu = g.standard_normal((I, H)) * 0.6, g.standard_normal((I, H)) * 0.6
    Wd = g.standard_normal((H, I))
    x = g.standard_normal((6, H)) * 2
    gg, uu, hh, oo = O.expert_ffn(x, Wg, Wu, Wd, 7.0)
    tx = torch.from_numpy(x)
    tg = tx @ torch.from_numpy(Wg).T
    tu = tx @ torch.from_numpy(Wu).T
    th = F.silu(torch.clamp(tg, max=7.0)) * torch.clamp(tu, min=-7.0, max=7.0)
    ref = th @ torch.from_numpy(Wd).T
    assert np.allclose(oo, ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.any(gg > 7) and np.any(np.abs(uu) > 7)  # the clamps were exercised
    # g >= 7 saturates to the constant silu(7)
    big = hh[(gg >= 7) & (np.abs(uu) < 7)]
    ratio = big / uu[(gg >= 7) & (np.abs(uu) < 7)]
    assert np.allclose(ratio, 7 / (1 + math.exp(-7)), rtol=1e-14)
    # clamp = inf is the unclamped form
    _, _, h_inf, _ = O.expert_ffn(x, Wg, Wu, Wd, np.inf)
    assert np.allclose(h_inf, (x @ Wg.T) / (1 + np.exp(-(x @ Wg.T))) * (x @ Wu.T), rtol=1e-13)


def test_moe_layer_identical_experts_and_k1():
    g = np.random.default_rng(9)
    H, I, E = 30, 10, 6
    x_bits = ti.f32_to_bf16_bits(g.standard_normal((5, H)).astype(np.float32))
    Wr = (g.standard_normal((E, H)) * 0.3).astype(np.float32)
    W = [g.standard_normal((I, H)).astype(np.float32), g.standard_normal((I, H)).astype(np.float32),
         g.standard_normal((H, I)).astype(np.float32)]
    # all experts identical: the weighted sum is one expert's output (weights sum to 1)
    res = O.moe_layer(x_bits, Wr, None, lambda e: W, k=4)
    x = O.bf16_to_f64(x_bits)
    deq = [O.dequantize(*O.ternarize_absmean(m)) for m in W]
    one = O.expert_ffn(x, *deq)[3]
    assert np.allclose(res["Y"], one, rtol=1e-12, atol=1e-12)
    # k = 1: the layer output is the selected expert's output
    Ws = [[(m * (e + 1)).astype(np.float32) for m in W] for e in range(E)]
    r1 = O.moe_layer(x_bits, Wr, None, lambda e: Ws[e], k=1)
    for t in range(5):
        e = int(r1["idx"][t, 0])
        d = [O.dequantize(*O.ternarize_absmean(m)) for m in Ws[e]]
        assert np.allclose(r1["Y"][t], O.expert_ffn(x[t:t + 1], *d)[3][0], rtol=1e-12)


def test_moe_layer_distinct_experts_dense_form():
    """The layer written densely over all experts, without grouping or slot
    positions: Y[t] = sum over the k selected experts e of
    softmax-over-the-selected(l)[e] * FFN_e(x_t), each FFN evaluated with
    torch's own linear / clamp / silu on the dequantized weights (codeinsider.com.br,
    "256 experts, 8 ativos": a weighted sum of the chosen experts' outputs).
    Distinct experts, k = 3 and unequal weights make any slot / weight / expert
    mix-up visible, as the swapped-weight check shows."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    g = np.random.default_rng(13)
    H, I, E, k, T = 24, 8, 6, 3, 7
    x_bits = ti.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    Wr = (g.standard_normal((E, H)) * 0.5).astype(np.float32)
    experts = [[g.standard_normal(sh).astype(np.float32) for sh in ((I, H), (I, H), (H, I))] for _ in range(E)]
    res = O.moe_layer(x_bits, Wr, None, lambda e: experts[e], k=k)
    x = O.bf16_to_f64(x_bits)
    logits = x @ Wr.astype(np.float64).T
    Y = np.zeros((T, H))
    Y_swapped = np.zeros((T, H))
    for t in range(T):
        order = np.argsort(-logits[t], kind="stable")
        chosen = order[:k]
        gaps = -np.diff(logits[t][order[:k + 1]])
        assert gaps.min() > 1e-6  # well separated: the selection is unambiguous
        p = np.exp(logits[t] - logits[t].max())
        w = p[chosen] / p[chosen].sum()
        assert np.ptp(w) > 0.05  # unequal weights
        outs = []
        for e in chosen:
            deq = [torch.from_numpy(O.dequantize(*O.ternarize_absmean(m))) for m in experts[e]]
            tx = torch.from_numpy(x[t:t + 1])
            th = F.silu(torch.clamp(tx @ deq[0].T, max=7.0)) * torch.clamp(tx @ deq[1].T, min=-7.0, max=7.0)
            o = th @ deq[2].T
            outs.append(o.numpy()[0])
        Y[t] = sum(wj * oj for wj, oj in zip(w, outs))
        Y_swapped[t] = w[1] * outs[0] + w[0] * outs[1] + sum(wj * oj for wj, oj in zip(w[2:], outs[2:]))
        assert np.array_equal(np.sort(res["idx"][t]), np.sort(chosen))
    assert np.allclose(res["Y"], Y, rtol=1e-12, atol=1e-12)
    # a weight paired with another slot's output would be caught
    assert O.max_normalized_error(Y_swapped, Y) > 1e-2


def test_combine_hand_example():
    Ob = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    w = np.array([[0.25, 0.75], [1.0, 0.0]])
    pos = np.array([2, 0, 1, 0])  # token 0 -> rows 2, 0 ; token 1 -> rows 1, 0
    Y = O.combine(Ob, w, pos)
    assert Y.tolist() == [[25.75, 51.5], [10.0, 20.0]]


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(10)
    v = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10.0 ** g.integers(-20, 20, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0], np.float32)])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_rne(v), ref)


def test_residual_rounding():
    x = ti.f32_to_bf16_bits(np.array([[1.0, 2.0]], np.float32))
    y = np.array([[2.0 ** -8, 2.0 ** -7 * 3]], np.float32)
    out = O.residual_bf16(x, y)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7: even mantissa -> 1.0 ; 2 + 3*2^-7 -> 2 + 2^-5
    assert O.bf16_to_f64(out).tolist() == [[1.0, 2.0 + 2.0 ** -5]]


def test_max_normalized_error():
    ref = np.array([[1.0, -4.0], [0.0, 0.0]])
    got = np.array([[1.0, -4.0 + 4e-5], [1e-3, 0.0]])
    assert abs(O.max_normalized_error(got, ref) - 1e-3) < 1e-15


# ----------------------------------------------------------- attention half (NEXT-3)
from oracle import attention_oracle as AO  # noqa: E402


def test_attention_census_and_pattern_match_pages():
    figs = _figs()
    H, I, E, L = int(figs["hidden"]), int(figs["moe_intermediate"]), int(figs["n_experts"]), int(figs["n_layers"])
    experts = 3 * I * H * E * L
    attn = L * (ti.ATTN_QKV_ROWS * H + H * AO.N_HEADS * AO.HEAD_DIM)
    assert ti.ATTN_QKV_ROWS * H + H * H == 2 * H * H + 2 * 512 * H == 10_485_760
    # the page's 19.58B ternary weights = experts + the attention projections
    assert round((experts + attn) / 1e9, 2) == figs["ternary_params"] / 1e9
    assert round(experts / 1e9, 2) == 19.33
    assert [l for l in range(L) if AO.is_global_layer(l)] == figs["global_layers"]
    assert AO.WINDOW == figs["sliding_window"] and AO.ROTARY_DIM == figs["partial_rotary_factor"] * AO.HEAD_DIM


def test_rope_matches_library_rotate_half():
    """Rotary on the first rot_dim dimensions with the rotate-half pairing, as the
    transformers library applies it (llama rotate_half on the rotated part, the
    rest passed through, inverse frequencies 1 / base^(2i / rot_dim))."""
    import torch
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    rng = np.random.default_rng(3)
    P, hd, rot, base = 40, 128, 64, 10000.0
    q = rng.standard_normal((2, P, hd))
    k = rng.standard_normal((1, P, hd))
    pos = np.arange(1000, 1000 + P)
    inv = 1.0 / (base ** (torch.arange(0, rot, 2, dtype=torch.float64) / rot))
    freqs = torch.outer(torch.tensor(pos, dtype=torch.float64), inv)
    emb = torch.cat([freqs, freqs], dim=-1)
    qt, kt = torch.tensor(q)[None], torch.tensor(k)[None]
    q_rot, k_rot = apply_rotary_pos_emb(qt[..., :rot], kt[..., :rot], emb.cos()[None], emb.sin()[None])
    want_q = torch.cat([q_rot, qt[..., rot:]], dim=-1)[0].numpy()
    want_k = torch.cat([k_rot, kt[..., rot:]], dim=-1)[0].numpy()
    assert np.allclose(AO.rope(q, pos), want_q, rtol=0, atol=1e-12)
    assert np.allclose(AO.rope(k, pos), want_k, rtol=0, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    for m, n, shift in ((5, 3, 1000), (0, 0, 77), (130000, 129600, -129000)):
        a = AO.rope(q, np.array([m]))[0] @ AO.rope(k, np.array([n]))[0]
        b = AO.rope(q, np.array([m + shift]))[0] @ AO.rope(k, np.array([n + shift]))[0]
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    r = AO.rope(q, np.array([12345]))
    assert np.array_equal(r[0, 64:], q[0, 64:])  # only the first half of the head turns
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12


def _tiny_attention(seed, P, global_layer, window=8):
    rng = np.random.default_rng(seed)
    H, nh, nkv, hd = 64, 8, 2, 16
    W = [rng.standard_normal(s) * 0.3 for s in ((nh * hd, H), (nkv * hd, H), (nkv * hd, H), (H, nh * hd))]
    x = ti.f32_to_bf16_bits(rng.standard_normal((P, H)).astype(np.float32))
    f = lambda xb: AO.attention_half(xb, *W, global_layer, n_heads=nh, n_kv=nkv, head_dim=hd, rot_dim=8,
                                     window=window)
    return x, W, f


def test_attention_matches_library_sdpa_with_explicit_mask():
    """Masking, scaling, softmax and the head-to-group map checked against
    torch's scaled_dot_product_attention on the oracle's own q, k, v."""
    import torch

    for global_layer in (False, True):
        x, W, f = _tiny_attention(5, 30, global_layer)
        r = f(x)
        q, k, v = (torch.tensor(r[n])[None] for n in ("q", "k", "v"))
        k, v = k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1)  # query head h reads group h // 4
        P = q.shape[2]
        mask = torch.tensor([[AO.visible(p, j, 0 if global_layer else 8) for j in range(P)] for p in range(P)])
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        got = r["attn"].reshape(P, 8, 16).transpose(1, 0, 2)
        assert np.allclose(got, want[0].numpy(), rtol=0, atol=1e-12)


def test_attention_window_locality():
    """A sliding query at p ignores every input older than p - window + 1 and
    depends on that one; a global query depends on position 0."""
    x, W, f = _tiny_attention(6, 40, global_layer=False, window=8)
    base = f(x)["o"][39]
    y = x.copy()
    y[:32] = ti.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((32, 64)).astype(np.float32))
    assert np.array_equal(f(y)["o"][39], base)
    y[32] = y[33]
    assert not np.allclose(f(y)["o"][39], base)
    xg, Wg, fg = _tiny_attention(6, 40, global_layer=True)
    yg = xg.copy()
    yg[0] = yg[1]
    assert not np.allclose(fg(yg)["o"][39], fg(xg)["o"][39])


def test_attention_special_cases():
    # one visible key: the output is its value vector, whatever the scores
    x, W, f = _tiny_attention(8, 1, global_layer=False)
    r = f(x)
    for h in range(8):
        assert np.allclose(r["attn"][0, 16 * h:16 * h + 16], r["v"][h // 4, 0], rtol=0, atol=1e-13)
    # global layer, identical inputs at every position: every key scores the same, output = the common value
    x, W, f = _tiny_attention(9, 12, global_layer=True)
    x[:] = x[0]
    r = f(x)
    for h in range(8):
        assert np.allclose(r["attn"][:, 16 * h:16 * h + 16], r["v"][h // 4, 0], rtol=0, atol=1e-12)
