"""GPU parity: every entry point of the C ABI against the CPU oracle on seeded
inputs. Integer and index results must match bit for bit; floating-point
results within a max normalized error (per row) of 2e-5."""
import math
import os

import numpy as np
import pytest

import oracle as O
import tmoe_inputs as ti

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2e-5


def say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module")
def tm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_moe_base_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits):
    return dev(np.ascontiguousarray(bits).view(np.int16))


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ws_bytes(n):
    return torch.zeros(max(int(n), 16), dtype=torch.uint8, device="cuda")


# --------------------------------------------------------------------- inputs
def test_synth_matches_host_generator(tm):
    for stream, n, first in [(ti.stream_id(1, 0, 0, 0), 512 * 2048, 0), (77, 1001, 12345)]:
        say(f"synth stream={stream} n={n}")
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        tm.synth_ih12(out, stream, first=first)
        assert np.array_equal(host(out), ti.ih12_normal(stream, n, first))
    r = torch.empty(256 * 2048, dtype=torch.float32, device="cuda")
    tm.synth_ih12(r, ti.stream_id(3, 0, 1023, ti.MAT_ROUTER), mult=float(ti.ROUTER_STD))
    assert np.array_equal(host(r).reshape(256, 2048), ti.router_matrix(3, 0))


# ------------------------------------------------------- ternarize / packing
@pytest.mark.parametrize("R,K,kind", [(512, 2048, "ih"), (2048, 512, "ih"), (33, 517, "normal"), (9, 23, "normal"),
                                      (5, 1, "normal")])
def test_ternarize_pack_device(tm, R, K, kind):
    say(f"ternarize_pack R={R} K={K} {kind}")
    g = np.random.default_rng(R + K)
    W = ti.ih12_normal(99, R * K).reshape(R, K) if kind == "ih" else g.standard_normal((R, K)).astype(np.float32)
    W[0, :2 if K > 1 else 1] = 0.0
    Kb = (K + 4) // 5
    P = torch.full((R, Kb + 3), 7, dtype=torch.uint8, device="cuda")
    s = torch.empty(R, dtype=torch.float32, device="cuda")
    tm.ternarize_pack(dev(W), P, s)
    t_ref, s_ref = O.ternarize_absmean(W)
    Ph = host(P)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(Ph[:, :Kb], O.pack_trits(t_ref))
    assert np.all(Ph[:, Kb:] == 7)  # bytes past ceil(K/5) untouched
    T = torch.empty((R, K), dtype=torch.int8, device="cuda")
    tm.unpack(P, K, T)
    assert np.array_equal(host(T), t_ref)


def test_ternarize_scale_sums_in_index_order(tm):
    """The scale's fp64 sum runs in index order, as the definition states: for
    |w| = (1, 2^-53, 2^-24, 2^-53) index order loses both 2^-53 terms to
    round-half-even and the mean 1/4 + 2^-26 rounds (half-even) to fp32 0.25,
    while pairing (1 + 2^-24) + (2^-53 + 2^-53) keeps 2^-52 and rounds up to
    0.25 + 2^-25. Rows: that pattern, scaled by powers of two and negated."""
    base = np.array([1.0, 2.0 ** -53, 2.0 ** -24, 2.0 ** -53])
    W = np.stack([base, 4.0 * base, -0.5 * base, base * np.array([1, -1, 1, -1])]).astype(np.float32)
    P = torch.empty((4, 1), dtype=torch.uint8, device="cuda")
    s = torch.empty(4, dtype=torch.float32, device="cuda")
    tm.ternarize_pack(dev(W), P, s)
    t_ref, s_ref = O.ternarize_absmean(W)
    assert np.array_equal(s_ref, np.array([0.25, 1.0, 0.125, 0.25], np.float32))
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(P)[:, 0], O.pack_trits(t_ref)[:, 0])


def test_unpack_all_codes(tm):
    codes = np.tile(np.arange(243, dtype=np.uint8), (3, 1))
    T = torch.empty((3, 243 * 5), dtype=torch.int8, device="cuda")
    tm.unpack(dev(codes), 243 * 5, T)
    assert np.array_equal(host(T), O.unpack_trits(codes, 243 * 5))


@pytest.mark.parametrize("R,K", [(1, 1), (9, 23), (16, 7), (33, 517), (512, 2048), (2048, 512), (17, 60), (3, 41)])
def test_tiled_layout_roundtrip(tm, R, K):
    say(f"tiled R={R} K={K}")
    g = np.random.default_rng(7 * R + K)
    t = g.integers(-1, 2, size=(R, K)).astype(np.int8)
    P = O.pack_trits(t)
    Pt = torch.empty(tm.tiled_bytes(R, K), dtype=torch.uint8, device="cuda")
    tm.repack_tiled(dev(P), K, Pt)
    T = torch.zeros((R, K), dtype=torch.int8, device="cuda")
    tm.unpack_tiled(Pt, R, K, T)
    assert np.array_equal(host(T), t)
    assert np.array_equal(host(Pt), _tiled_image(t))


def _tiled_image(t):
    """The tiled byte image of trits t [R][K], built from the layout's
    description (16-row tiles, four quarters of 5Q inputs, steps of 8 bytes
    whose byte 2p+h holds inputs 40*step + 10p + 2q + h of the quarter)."""
    R, K = t.shape
    Q = -(-(-(-K // 5)) // 4)
    Q += Q % 2
    Q = max(Q, 2)
    F, r = Q // 8, Q % 8
    tile_bytes = 64 * Q
    nt = -(-R // 16)
    out = np.zeros(nt * tile_bytes, dtype=np.uint8)
    tp = np.zeros((nt * 16, 20 * Q), dtype=np.int64)
    tp[:R, :K] = t
    for lane in range(64):
        i, g = lane & 15, lane >> 4
        for b in range(Q):
            if b < 8 * F:
                s, bb = b // 8, b % 8
                off = s * 512 + lane * 8 + bb
            else:
                s, bb = F, b - 8 * F
                if r >= 4:
                    off = 512 * F + (lane * 4 + bb if bb < 4 else 256 + lane * 2 + bb - 4)
                else:
                    off = 512 * F + lane * 2 + bb
            ks = [5 * Q * g + 40 * s + 10 * (bb >> 1) + 2 * q + (bb & 1) for q in range(5)]
            rows = np.arange(nt) * 16 + i
            code = sum((tp[rows, k] + 1) * 3 ** q for q, k in enumerate(ks))
            out[np.arange(nt) * tile_bytes + off] = code
    return out


# ------------------------------------------------------------- ternary linear
def _linear(tm, t, s, x_bits):
    N, K = t.shape
    T = x_bits.shape[0]
    Pt = torch.empty(tm.tiled_bytes(N, K), dtype=torch.uint8, device="cuda")
    tm.repack_tiled(dev(O.pack_trits(t)), K, Pt)
    Y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = ws_bytes(tm.linear_workspace_bytes(T, K))
    tm.ternary_linear(Pt, dev(s), N, K, bf16_dev(x_bits), Y, ws)
    return host(Y)


@pytest.mark.parametrize("N,K,T", [(512, 2048, 4), (512, 2048, 1), (512, 2048, 37), (2048, 512, 5), (9, 23, 3),
                                   (33, 517, 17), (20, 60, 2), (1, 1, 1)])
def test_ternary_linear_integer_inputs_exact(tm, N, K, T):
    # integer activations and power-of-two scales make every partial sum exact
    say(f"linear exact N={N} K={K} T={T}")
    g = np.random.default_rng(N + K + T)
    t = g.integers(-1, 2, size=(N, K)).astype(np.int8)
    s = (2.0 ** g.integers(-4, 4, size=N)).astype(np.float32)
    xb = ti.integer_activations(N + T, T, K)
    Y = _linear(tm, t, s, xb)
    ref = O.ternary_linear(t, s, O.bf16_to_f64(xb)).astype(np.float32)
    assert np.array_equal(Y, ref)


@pytest.mark.parametrize("T", [4, 1, 37, 256])
def test_ternary_linear_config1(tm, T):
    # 2048 -> 512, weights N(0,1) (Irwin-Hall) absmean-ternarized on the device, bf16 N(0,1) input
    say(f"linear config1 T={T}")
    N, K = 512, 2048
    W = torch.empty(N * K, dtype=torch.float32, device="cuda")
    tm.synth_ih12(W, ti.stream_id(1, 0, 0, ti.MAT_GATE))
    P = torch.empty((N, 410), dtype=torch.uint8, device="cuda")
    s = torch.empty(N, dtype=torch.float32, device="cuda")
    tm.ternarize_pack(W.view(N, K), P, s)
    Pt = torch.empty(tm.tiled_bytes(N, K), dtype=torch.uint8, device="cuda")
    tm.repack_tiled(P, K, Pt)
    xb = ti.activations(1, T)
    Y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    tm.ternary_linear(Pt, s, N, K, bf16_dev(xb), Y, ws_bytes(tm.linear_workspace_bytes(T, K)))
    t_ref, s_ref = O.ternarize_absmean(ti.linear_matrix(1))
    Tt = torch.empty((N, K), dtype=torch.int8, device="cuda")
    tm.unpack_tiled(Pt, N, K, Tt)
    assert np.array_equal(host(Tt), t_ref)
    ref = O.ternary_linear(t_ref, s_ref, O.bf16_to_f64(xb))
    err = O.max_normalized_error(host(Y), ref)
    say(f"  max normalized error {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("N,K,T,ldp", [(512, 2048, 4, 410), (300, 1000, 37, 208), (17, 2048, 1, 416)])
def test_ternary_linear_packed(tm, N, K, T, ldp):
    """The canonical-byte entry point: the host-packed bytes of oracle trits
    (row stride ldp, ragged row tiles, K not a multiple of 5 or of the step)
    give the oracle's product, and the same Y bit for bit as repacking once
    and calling the tiled entry point."""
    say(f"linear packed N={N} K={K} T={T} ldp={ldp}")
    g = np.random.default_rng(N * 7 + K + T)
    t, s = O.ternarize_absmean(g.standard_normal((N, K)).astype(np.float32))
    Ph = O.pack_trits(t, ldp)
    xb = ti.activations(3, T, K)
    x = O.bf16_to_f64(xb)
    P = torch.from_numpy(Ph).cuda()
    sd = dev(s.astype(np.float32))
    Xd = bf16_dev(xb)
    Y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    tm.ternary_linear_packed(P, sd, K, Xd, Y, ws_bytes(tm.linear_packed_workspace_bytes(N, K, T)))
    Pt = torch.empty(tm.tiled_bytes(N, K), dtype=torch.uint8, device="cuda")
    tm.repack_tiled(P, K, Pt)
    Y2 = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    tm.ternary_linear(Pt, sd, N, K, Xd, Y2, ws_bytes(tm.linear_workspace_bytes(T, K)))
    assert np.array_equal(host(Y), host(Y2))
    err = O.max_normalized_error(host(Y), O.ternary_linear(t, s.astype(np.float32), x))
    say(f"  max normalized error {err:.2e}")
    assert err <= TOL


def test_ternary_linear_streamed(tm):
    """The streamed variant of the 2048 -> 512 linear: 2048 distinct matrices
    stacked into one 1,048,576 x 2048 operand (436 MB packed), 4 tokens, in the
    launch the benchmark times (one token tile, full-K row tiles per
    wavefront); sampled matrices against the oracle, every output finite."""
    from ternary_weight_moe_base_amd import synthetic
    mats, N, K, T = 2048, 2048 * 512, 2048, 4
    say(f"linear streamed N={N} K={K} T={T}")
    Pt, s = synthetic.streamed_linear(1, mats)
    xb = ti.activations(1, T)
    Y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    tm.ternary_linear(Pt, s, N, K, bf16_dev(xb), Y, ws_bytes(tm.linear_workspace_bytes(T, K)))
    Yh = host(Y)
    assert np.isfinite(Yh).all()
    x = O.bf16_to_f64(xb)
    for q in (0, 1, 1023, 2047):
        t_ref, s_ref = O.ternarize_absmean(ti.expert_matrix(1, q // 1024, q % 1024, ti.MAT_GATE))
        ref = O.ternary_linear(t_ref, s_ref, x)
        err = O.max_normalized_error(Yh[:, q * 512:(q + 1) * 512], ref)
        say(f"  matrix {q}: max normalized error {err:.2e}")
        assert err <= TOL


# --------------------------------------------------------------------- router
def _router(tm, xb, Wr, bias, k, with_logits=True):
    """Router through the C ABI. From 1024 tokens on, a call that does not
    ask for the logits takes the bf16 matrix-core candidate path (fp64
    recompute of the candidates); one that asks for them takes the fp64
    matrix-core logits (as every call from 65 to 1023 tokens does)."""
    T, H = xb.shape
    E = Wr.shape[0]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nf = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    tm.router_topk(bf16_dev(xb), dev(Wr), None if bias is None else dev(bias), k, idx, w,
                   ws_bytes(tm.router_workspace_bytes(T, E)), logits=lg, n_fixup=nf)
    return host(idx), host(w), int(host(nf)[0]), host(lg) if with_logits else None


@pytest.mark.parametrize("cfg,T,bias_kind,with_logits", [
    (2, 1, None, True), (3, 64, "zipf", True), (4, 4096, "uniform", True), (5, 256, None, True),
    (4, 4096, "uniform", False), (5, 256, None, False), (3, 65, "zipf", False), (5, 1024, None, False)])
def test_router_parity(tm, cfg, T, bias_kind, with_logits):
    say(f"router cfg={cfg} T={T} logits={with_logits}")
    xb = ti.activations(cfg, T)
    Wr = ti.router_matrix(cfg, 0)
    b = ti.router_bias(cfg, bias_kind)
    idx, w, nfix, lg = _router(tm, xb, Wr, b, 8, with_logits)
    ridx, rw, rL, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, 8)
    say(f"  exact-path tokens: {nfix} of {T}")
    assert nfix == 0  # fp64 values separate every ranking of these inputs
    assert np.array_equal(idx, ridx)
    assert O.max_normalized_error(w, rw) <= TOL
    if with_logits:
        assert O.max_normalized_error(lg, rL) <= TOL
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("T,with_logits", [(40, True), (8, True), (1100, False), (300, True)])
def test_router_ties_take_exact_path(tm, T, with_logits):
    # exactly equal logits cannot be certified by the error bound: those tokens
    # are recomputed in double-double and the tie goes to the lower index
    H, E = 2048, 256
    xb = ti.activations(9, T)
    Wr = ti.router_matrix(9, 0).copy()
    Wr[200] = Wr[17]
    Wr[201] = Wr[17]
    b = np.zeros(E, np.float32)
    b[[17, 200, 201]] = 5.0
    idx, w, nfix, _ = _router(tm, xb, Wr, b, 8, with_logits)
    ridx, rw, rL, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, 8)
    # tokens whose exact top 9 holds the tie (a token whose own logits push
    # the trio below its 9th largest is certified without it)
    tied = np.array([17 in np.argsort(-row, kind="stable")[:9] for row in rL])
    say(f"  tokens with the tie in their top 9: {tied.sum()} of {T}; double-double tokens: {nfix}")
    assert nfix == tied.sum()
    assert np.array_equal(idx, ridx)
    for row in idx[tied]:  # the tied experts come in index order
        trio = [int(e) for e in row if e in (17, 200, 201)]
        assert trio == sorted(trio)
    assert O.max_normalized_error(w, rw) <= TOL


def _near_tie_router(seed):
    # three equal router rows whose biases differ by one and two fp32 ulps of
    # 5.0: the logits differ by ~5e-7, far below fp32 resolution of their
    # ordering near 5 but far above the fp64 error bound, and the value order
    # (250 > 99 > 3) is the reverse of the index order
    Wr = ti.router_matrix(seed, 0).copy()
    Wr[99] = Wr[3]
    Wr[250] = Wr[3]
    b = np.zeros(256, np.float32)
    b[3] = 5.0
    b[99] = np.nextafter(np.float32(5.0), np.float32(6.0))
    b[250] = np.nextafter(b[99], np.float32(6.0))
    return Wr, b


@pytest.mark.parametrize("T,with_logits", [(40, True), (8, True), (1100, False), (300, True)])
def test_router_near_ties_certified_in_fp64(tm, T, with_logits):
    # logits that share an fp32 bucket but are separated in fp64: certified
    # without the double-double recompute, in value order (on the candidate
    # path the three are candidates of every token and their fp64 values
    # decide)
    xb = ti.activations(10, T)
    Wr, b = _near_tie_router(10)
    idx, w, nfix, _ = _router(tm, xb, Wr, b, 8, with_logits)
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, 8)
    assert nfix == 0
    assert np.array_equal(idx, ridx)
    for row in idx:  # the three come in value order (the reverse of index order)
        trio = [int(e) for e in row if e in (3, 99, 250)]
        assert trio == [250, 99, 3][:len(trio)]
    assert (idx[:, 0] == 250).mean() > 0.9
    assert O.max_normalized_error(w, rw) <= TOL


@pytest.mark.parametrize("k,E,H,T,with_logits", [
    (1, 256, 2048, 33, True), (16, 256, 2048, 9, True), (8, 64, 256, 100, True), (4, 1000, 512, 7, True),
    (64 // 8, 8, 256, 5, True), (8, 200, 512, 1100, True), (4, 72, 256, 1031, True),
    (8, 64, 256, 1100, False), (8, 200, 512, 1100, False), (4, 72, 256, 1031, False), (16, 1000, 4096, 1030, False),
    (1, 256, 1024, 1077, False), (8, 8, 256, 1070, False), (8, 256, 2048, 1024, False)])
def test_router_shapes(tm, k, E, H, T, with_logits):
    say(f"router k={k} E={E} H={H} T={T} logits={with_logits}")
    g = np.random.default_rng(k + E + H + T)
    xb = ti.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    Wr = (g.standard_normal((E, H)) * 0.02).astype(np.float32)
    b = g.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, w, _, _ = _router(tm, xb, Wr, b, k, with_logits)
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, k)
    assert np.array_equal(idx, ridx)
    assert O.max_normalized_error(w, rw) <= TOL


# ------------------------------------------------------------------- grouping
def _group(tm, idx, E):
    T, k = idx.shape
    out = [torch.full((n,), -9, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k, T * k)]
    ws = ws_bytes(tm.group_workspace_bytes(T, k, E))
    tm.group_by_expert(dev(idx.astype(np.int32)), E, *out, ws=ws)
    return [host(o) for o in out]


@pytest.mark.parametrize("T,k,E,mode", [(1, 8, 256, "rand"), (7, 8, 256, "rand"), (64, 8, 256, "zipf"),
                                        (256, 8, 256, "rand"), (257, 8, 256, "rand"), (1000, 1, 64, "rand"),
                                        (4096, 8, 256, "rand"), (300, 16, 1000, "rand"), (600, 8, 256, "one"),
                                        (50, 40, 128, "rand"), (700, 12, 64, "rand"), (300, 20, 256, "rand"),
                                        (16384, 8, 256, "rand"), (16640, 8, 256, "rand")])
def test_grouping_parity(tm, T, k, E, mode):
    """One workgroup (T <= 256), count + scatter with the scan folded in (up to
    64 blocks of 256 tokens; T = 16384: exactly 64) and count + scan + scatter
    (T = 16640: 65 blocks) against the oracle's grouping."""
    say(f"group T={T} k={k} E={E} {mode}")
    g = np.random.default_rng(T * 31 + k + E)
    if mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        idx = np.stack([g.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)])
    if mode == "one":
        idx[:, 0] = 5  # one expert holds every token
        for t in range(T):
            while 5 in idx[t, 1:]:
                idx[t, 1:][idx[t, 1:] == 5] = g.integers(6, E)
    got = _group(tm, idx, E)
    ref = O.group_by_expert(idx, E)
    for a, b_ in zip(got, ref):
        assert np.array_equal(a, b_)


# ---------------------------------------------------------------- whole layer
_EXPERT_CACHE = {}


def _raw_expert(cfg, layer, e):
    key = (cfg, layer, e)
    if key not in _EXPERT_CACHE:
        _EXPERT_CACHE[key] = tuple(ti.expert_matrix(cfg, layer, e, m) for m in (0, 1, 2))
    return _EXPERT_CACHE[key]


def _prefetch_experts(cfg, layer, experts):
    """Draws the raw fp32 matrices of `experts` on the host, in parallel (the
    generator releases the interpreter lock)."""
    import concurrent.futures
    todo = [int(e) for e in experts if (cfg, layer, int(e)) not in _EXPERT_CACHE]
    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        list(ex.map(lambda e: _raw_expert(cfg, layer, e), todo))


def _scaled(xb, scale):
    """bf16 bit patterns of scale * x (scale a power of two: exact)."""
    if scale == 1:
        return xb
    return ti.f32_to_bf16_bits(ti.bf16_bits_to_f32(xb) * np.float32(scale))


@pytest.fixture(scope="module")
def layers():
    from ternary_weight_moe_base_amd import synthetic
    cache = {}

    def get(cfg, layer, bias):
        key = (cfg, layer, bias)  # the routing bias is part of the device layer
        if key not in cache:
            say(f"building layer cfg={cfg} layer={layer} bias={bias} on the device")
            cache[key] = synthetic.build_layer(cfg, layer, bias)
            torch.cuda.synchronize()
        return cache[key]
    return get


def _run_layer(tm, W, xb, clamp=7.0):
    T = xb.shape[0]
    k = W.top_k
    Y = torch.empty((T, W.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    pos = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ws_bytes(tm.moe_workspace_bytes(T, W))
    tm.moe_forward(W, bf16_dev(xb), Y, ws, clamp=clamp, idx=idx, w=w, pos=pos, n_fixup=nf)
    return dict(Y=host(Y), idx=host(idx), w=host(w), pos=host(pos), nfix=int(host(nf)[0]))


# (cfg, T, bias, clamp, input scale): both clamp modes; without the clamp,
# inputs x4 drive |h| past the fp16 range (up to ~1e5), and inputs x2^-10 make
# every h tiny (~1e-6): the down projection's per-pair scaling must hold both.
@pytest.mark.parametrize("cfg,T,bias_kind,clamp,scale", [
    (2, 1, None, 7.0, 1), (2, 1, None, math.inf, 1), (3, 64, "zipf", 7.0, 1), (3, 64, "zipf", math.inf, 1),
    (2, 5, None, 7.0, 1), (2, 4, None, 7.0, 1), (3, 16, "zipf", 7.0, 1), (5, 256, None, 7.0, 1),
    (2, 1, None, math.inf, 4), (3, 64, "zipf", math.inf, 4), (2, 1, None, 7.0, 2.0 ** -10),
    (5, 256, None, 7.0, 2.0 ** -10), (2, 3, None, math.inf, 16)])
def test_layer_parity(tm, layers, cfg, T, bias_kind, clamp, scale):
    say(f"layer cfg={cfg} T={T} clamp={clamp} input scale={scale}")
    W = layers(cfg, 0, bias_kind)
    xb = _scaled(ti.activations(cfg, T), scale)
    got = _run_layer(tm, W, xb, clamp)
    Wr, bias = ti.router_matrix(cfg, 0), ti.router_bias(cfg, bias_kind)
    _prefetch_experts(cfg, 0, np.unique(O.router_topk(O.bf16_to_f64(xb), Wr, bias, 8)[0]))
    ref = O.moe_layer(xb, Wr, bias, lambda e: _raw_expert(cfg, 0, e), k=8, clamp=clamp)
    say(f"  max |h| {np.abs(ref['H']).max():.3e}, min |h| {np.abs(ref['H']).min():.3e}")
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["pos"], ref["pos"])
    err = O.max_normalized_error(got["Y"], ref["Y"])
    say(f"  Y max normalized error {err:.2e} (experts hit: {int((ref['counts'] > 0).sum())})")
    assert err <= TOL
    # the step-by-step ABI gives the same layer, and its intermediates match too
    T_, k = xb.shape[0], 8
    E = 256
    idx = dev(got["idx"])
    g = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T_ * k, T_ * k, T_ * k)]
    tm.group_by_expert(idx, E, *g, ws=ws_bytes(tm.group_workspace_bytes(T_, k, E)))
    O_ = torch.empty((T_ * k, 2048), dtype=torch.float32, device="cuda")
    Hh = torch.empty((T_ * k, 512), dtype=torch.float32, device="cuda")
    tm.expert_ffn(W, bf16_dev(xb), g[1], g[2], O_, ws_bytes(tm.ffn_workspace_bytes(T_, W)), clamp=clamp, Hout=Hh)
    Y2 = torch.empty((T_, 2048), dtype=torch.float32, device="cuda")
    tm.combine(O_, dev(got["w"]), g[4], Y=Y2)
    assert O.max_normalized_error(host(Hh), ref["H"]) <= TOL
    assert O.max_normalized_error(host(O_), ref["O"]) <= TOL
    if T_ > 16:
        assert np.array_equal(host(Y2), got["Y"])  # the layer runs these same kernels
    else:
        # decode path: the combine is fused into the down kernel (another fp32 summation order)
        assert O.max_normalized_error(host(Y2), got["Y"]) <= 1e-6


@pytest.mark.parametrize("E,k,T", [(8, 8, 3), (8, 8, 6), (8, 2, 16), (16, 4, 9), (16, 4, 17), (16, 12, 3),
                                   (32, 16, 2), (64, 8, 200), (128, 8, 130)])
def test_layer_few_experts(tm, E, k, T):
    """Edge cases of both paths: more (token, slot) pairs than experts, every
    expert hit, up to 16 pairs per tile; on the decode path (T <= 3) the fused
    combine (T k <= 32) and the separate one (T k > 32); batches of 1024 or
    more pairs (eight-wavefront gate/up workgroups, several tiles per expert)."""
    from ternary_weight_moe_base_amd import synthetic
    say(f"layer E={E} k={k} T={T}")
    cfg = 2
    W = synthetic.build_layer(cfg, 0, None, experts=E, top_k=k)
    xb = ti.activations(cfg, T)
    got = _run_layer(tm, W, xb)
    ref = O.moe_layer(xb, ti.router_matrix(cfg, 0)[:E], None, lambda e: _raw_expert(cfg, 0, e), k=k)
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["pos"], ref["pos"])
    err = O.max_normalized_error(got["Y"], ref["Y"])
    say(f"  Y max normalized error {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("E,k,T", [(8, 2, 600), (16, 4, 333)])
def test_layer_token_blocked(tm, E, k, T):
    """Many pairs per expert (the token-blocked gate/up path): every output of
    the layer, and h and the expert outputs of the step-by-step ABI."""
    from ternary_weight_moe_base_amd import synthetic
    say(f"layer token-blocked E={E} k={k} T={T}")
    cfg = 4
    W = synthetic.build_layer(cfg, 0, None, experts=E, top_k=k)
    xb = ti.activations(cfg, T)
    got = _run_layer(tm, W, xb)
    ref = O.moe_layer(xb, ti.router_matrix(cfg, 0)[:E], None, lambda e: _raw_expert(cfg, 0, e), k=k)
    assert np.array_equal(got["idx"], ref["idx"])
    assert np.array_equal(got["pos"], ref["pos"])
    say(f"  pairs per expert: {np.bincount(ref['idx'].ravel(), minlength=E).tolist()}")
    err = O.max_normalized_error(got["Y"], ref["Y"])
    say(f"  Y max normalized error {err:.2e}")
    assert err <= TOL
    g = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k, T * k)]
    tm.group_by_expert(dev(got["idx"]), E, *g, ws=ws_bytes(tm.group_workspace_bytes(T, k, E)))
    O_ = torch.empty((T * k, 2048), dtype=torch.float32, device="cuda")
    Hh = torch.empty((T * k, 512), dtype=torch.float32, device="cuda")
    tm.expert_ffn(W, bf16_dev(xb), g[1], g[2], O_, ws_bytes(tm.ffn_workspace_bytes(T, W)), Hout=Hh)
    assert O.max_normalized_error(host(Hh), ref["H"]) <= TOL
    assert O.max_normalized_error(host(O_), ref["O"]) <= TOL


def _grouped_ffn_reference(cfg, layer, x, sorted_token, offsets, clamps):
    """Oracle expert FFN of every grouped pair, expert by expert in parallel
    threads: {clamp: (H, O)} in grouped order (the same per-expert steps as the
    oracle's moe_layer: absmean ternarization, dense dequantized weights,
    expert_ffn)."""
    import concurrent.futures
    P = len(sorted_token)
    out = {c: (np.zeros((P, 512)), np.zeros((P, 2048))) for c in clamps}

    def one(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            return
        deq = [O.dequantize(*O.ternarize_absmean(m)) for m in _raw_expert(cfg, layer, e)]
        xe = x[sorted_token[lo:hi]]
        for c in clamps:
            _, _, h, o = O.expert_ffn(xe, *deq, c)
            out[c][0][lo:hi], out[c][1][lo:hi] = h, o
    with concurrent.futures.ThreadPoolExecutor(16) as ex:
        list(ex.map(one, range(len(offsets) - 1)))
    return out


def test_layer_prefill_every_row(tm, layers):
    """Prefill of 4096 tokens (uniform routing bias), in both clamp modes:
    router and grouping on every token; Y of the layer on every one of the 4096
    rows; h and the expert outputs of all 32,768 pairs through the step-by-step
    ABI (tmoe_expert_ffn), all against the oracle."""
    cfg, T, k, E = 4, 4096, 8, 256
    W = layers(cfg, 0, "uniform")
    xb = ti.activations(cfg, T)
    Wr, b = ti.router_matrix(cfg, 0), ti.router_bias(cfg, "uniform")
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, 8)
    counts, offsets, st, ss, pos = O.group_by_expert(ridx, E)
    say(f"layer prefill T=4096: expert counts min {counts.min()} max {counts.max()} mean {counts.mean():.1f}")
    _prefetch_experts(cfg, 0, range(E))
    ref = _grouped_ffn_reference(cfg, 0, O.bf16_to_f64(xb), st, offsets, (7.0, math.inf))
    g = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k, T * k)]
    tm.group_by_expert(dev(ridx.astype(np.int32)), E, *g, ws=ws_bytes(tm.group_workspace_bytes(T, k, E)))
    assert np.array_equal(host(g[1]), offsets) and np.array_equal(host(g[2]), st)
    for clamp in (7.0, math.inf):
        got = _run_layer(tm, W, xb, clamp)
        assert np.array_equal(got["idx"], ridx)
        assert np.array_equal(got["pos"], pos)
        Href, Oref = ref[clamp]
        Yref = O.combine(Oref, rw, pos)
        err = O.max_normalized_error(got["Y"], Yref)
        say(f"  clamp={clamp}: Y max normalized error over all {T} rows {err:.2e}")
        assert err <= TOL
        O_ = torch.empty((T * k, 2048), dtype=torch.float32, device="cuda")
        Hh = torch.empty((T * k, 512), dtype=torch.float32, device="cuda")
        tm.expert_ffn(W, bf16_dev(xb), g[1], g[2], O_, ws_bytes(tm.ffn_workspace_bytes(T, W)), clamp=clamp, Hout=Hh)
        eh, eo = O.max_normalized_error(host(Hh), Href), O.max_normalized_error(host(O_), Oref)
        say(f"  clamp={clamp}: h error {eh:.2e}, expert outputs error {eo:.2e} over all {T * k} pairs")
        assert eh <= TOL and eo <= TOL
        del O_, Hh


@pytest.mark.parametrize("T,bias_kind", [(1023, "uniform"), (1024, "uniform"), (2048, "zipf")])
def test_layer_at_the_prefill_switch(tm, layers, T, bias_kind):
    """Both sides of the 1024-token switch, where the router moves from the
    fp64 matrix-core logits (+ the top-k kernel) to the bf16 candidates refined
    in fp64, and the expert kernels from 16-pair tiles to the token-blocked
    form (T k >= 32 E): idx, pos and Y on every row against the oracle. The
    Zipf-routed case gives the token-blocked kernels one expert with dozens of
    full blocks next to experts with a single partial block or none."""
    cfg, k, E = 4, 8, 256
    W = layers(cfg, 0, bias_kind)
    xb = ti.activations(cfg, T)
    Wr, b = ti.router_matrix(cfg, 0), ti.router_bias(cfg, bias_kind)
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, k)
    counts, offsets, st, ss, pos = O.group_by_expert(ridx, E)
    say(f"layer T={T}: {T * k} pairs, expert counts min {counts.min()} max {counts.max()}")
    _prefetch_experts(cfg, 0, range(E))
    Href, Oref = _grouped_ffn_reference(cfg, 0, O.bf16_to_f64(xb), st, offsets, (7.0,))[7.0]
    got = _run_layer(tm, W, xb, 7.0)
    say(f"  tokens recomputed in double-double: {got['nfix']}")
    assert np.array_equal(got["idx"], ridx)
    assert np.array_equal(got["pos"], pos)
    assert O.max_normalized_error(got["w"], rw) <= TOL
    err = O.max_normalized_error(got["Y"], O.combine(Oref, rw, pos))
    say(f"  Y max normalized error over all {T} rows {err:.2e}")
    assert err <= TOL


def test_layer_is_deterministic(tm, layers):
    W = layers(3, 0, "zipf")
    xb = ti.activations(3, 64)
    a = _run_layer(tm, W, xb)
    b = _run_layer(tm, W, xb)
    for key in ("Y", "idx", "w", "pos"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


def test_layer_workspace_reuse(tm, layers):
    # one workspace, alternating sizes: whatever a call leaves there does not change the next call
    W = layers(2, 0, None)
    ws = ws_bytes(tm.moe_workspace_bytes(16, W))
    outs = {}
    for rep in range(3):
        for T in (1, 16, 5):
            xb = ti.activations(7, T)
            Y = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
            idx = torch.empty((T, 8), dtype=torch.int32, device="cuda")
            tm.moe_forward(W, bf16_dev(xb), Y, ws, idx=idx)
            got = (host(Y), host(idx))
            if rep == 0:
                outs[T] = got
                ridx, _, _, _ = O.router_topk(O.bf16_to_f64(xb), ti.router_matrix(2, 0), None, 8)
                assert np.array_equal(got[1], ridx)
            else:
                assert np.array_equal(got[0], outs[T][0]) and np.array_equal(got[1], outs[T][1])


@pytest.mark.parametrize("T", [1, 3, 64, 300])
def test_layer_workspace_needs_no_zero_fill(tm, layers, T):
    """A workspace full of 0xFF bytes (NaN as fp64, -1 as int32) gives the
    zero-filled workspace's result bit for bit, and no token takes the
    double-double path (a bound slot read before its write would be NaN and
    fail every certification)."""
    say(f"layer with a 0xFF-filled workspace T={T}")
    W = layers(2, 0, None)
    xb = ti.activations(11, T)
    ref = _run_layer(tm, W, xb)
    n = tm.moe_workspace_bytes(T, W)
    ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda")
    Y = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    nf = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for rep in range(2):
        tm.moe_forward(W, bf16_dev(xb), Y, ws, idx=idx, n_fixup=nf)
        assert np.array_equal(host(Y), ref["Y"]), rep
        assert np.array_equal(host(idx), ref["idx"]), rep
        assert int(host(nf)[0]) == ref["nfix"] == 0, rep


def test_layer_decode_ties(tm, layers):
    # the fused decode front end with exactly tied router rows (exact path inside the kernel)
    from ternary_weight_moe_base_amd import synthetic
    W = layers(2, 0, None)
    Wr = W.tensors[0].clone()
    Wr[99] = Wr[3]
    Wr[250] = Wr[3]
    b = torch.zeros(256, dtype=torch.float32, device="cuda")
    b[[3, 99, 250]] = 5.0
    W2 = type(W)(Wr, b, *W.tensors[2:], top_k=8)
    xb = ti.activations(11, 6)
    got = _run_layer(tm, W2, xb)
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), host(Wr), host(b), 8)
    assert got["nfix"] == 6
    assert np.array_equal(got["idx"], ridx)
    assert np.all(got["idx"][:, :3] == [3, 99, 250])


@pytest.mark.parametrize("T", [1, 6])
def test_layer_decode_near_ties(tm, layers, T):
    # the decode front end with logits separated only in fp64 (value order
    # reverses index order): certified in fp64, no double-double recompute
    W = layers(2, 0, None)
    Wr, b = _near_tie_router(2)
    W2 = type(W)(dev(Wr), dev(b), *W.tensors[2:], top_k=8)
    xb = ti.activations(12, T)
    got = _run_layer(tm, W2, xb)
    ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), Wr, b, 8)
    assert got["nfix"] == 0
    assert np.array_equal(got["idx"], ridx)
    assert np.all(got["idx"][:, :3] == [250, 99, 3])
    assert O.max_normalized_error(got["w"], rw) <= TOL


def test_layer_empty_batch(tm, layers):
    W = layers(2, 0, None)
    Y = torch.empty((0, 2048), dtype=torch.float32, device="cuda")
    tm.moe_forward(W, torch.empty((0, 2048), dtype=torch.int16, device="cuda"), Y, ws_bytes(16))


def test_stack_teacher_forced(tm, layers):
    # 24-layer stack workload, first layers: the oracle's layer l consumes the
    # GPU's residual stream X_l (teacher forcing); Y of layer 1 on every one of
    # the 256 tokens (grouped oracle experts), and two tokens of each layer
    # through the oracle's per-token loop
    cfg, T = 5, 256
    xb = ti.activations(cfg, T)
    for layer in range(2):
        W = layers(cfg, layer, None)
        X = bf16_dev(xb)
        Y = torch.empty((T, 2048), dtype=torch.float32, device="cuda")
        Xn = torch.empty_like(X)
        idx = torch.empty((T, 8), dtype=torch.int32, device="cuda")
        w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
        tm.moe_forward(W, X, Y, ws_bytes(tm.moe_workspace_bytes(T, W)), idx=idx, w=w, resid_out=Xn)
        Yh, idxh, xn = host(Y), host(idx), host(Xn).view(np.uint16)
        ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), ti.router_matrix(cfg, layer), None, 8)
        assert np.array_equal(idxh, ridx)
        # the residual stream is bf16(x + y) of the GPU's own y
        assert np.array_equal(xn, O.residual_bf16(xb, Yh))
        x = O.bf16_to_f64(xb)
        if layer == 1:  # the layer fed by the GPU's own residual stream: every token
            _, offsets, st, _, pos = O.group_by_expert(ridx, 256)
            _prefetch_experts(cfg, layer, range(256))
            Oref = _grouped_ffn_reference(cfg, layer, x, st, offsets, (7.0,))[7.0][1]
            err = O.max_normalized_error(Yh, O.combine(Oref, rw, pos))
            say(f"  stack layer {layer}: Y max normalized error over all {T} tokens {err:.2e}")
            assert err <= TOL
        for t in (3, 200):
            y = np.zeros(2048)
            for j in range(8):
                deq = [O.dequantize(*O.ternarize_absmean(m)) for m in _raw_expert(cfg, layer, int(ridx[t, j]))]
                y += rw[t, j] * O.expert_ffn(x[t:t + 1], *deq)[3][0]
            err = O.max_normalized_error(Yh[t:t + 1], y[None])
            say(f"  stack layer {layer} token {t}: max normalized error {err:.2e}")
            assert err <= TOL
        xb = xn


def test_stack_decode_one_token(tm, layers):
    """One token through all 24 layers of the stack workload, each layer's
    output feeding the next through the bf16 residual stream (the one-token
    decode chain): every layer's top-8 and residual checked, Y against the
    oracle (teacher-forced) on sampled layers; the same chain captured in one
    HIP graph and replayed gives the eager result bit for bit."""
    cfg, L = 5, 24
    xb0 = ti.activations(cfg, 3)[2:3]
    Ws = [layers(cfg, l, None) for l in range(L)]
    ws = ws_bytes(tm.moe_workspace_bytes(1, Ws[0]))
    Y = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, 1, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((L, 1, 8), dtype=torch.float32, device="cuda")
    xs = [bf16_dev(xb0)] + [torch.empty((1, 2048), dtype=torch.int16, device="cuda") for _ in range(L)]
    xb = xb0
    for l in range(L):
        tm.moe_forward(Ws[l], xs[l], Y, ws, idx=idx[l], w=w[l], resid_out=xs[l + 1])
        Yh, xn = host(Y), host(xs[l + 1]).view(np.uint16)
        ridx, rw, _, _ = O.router_topk(O.bf16_to_f64(xb), ti.router_matrix(cfg, l), None, 8)
        assert np.array_equal(host(idx[l]), ridx), l
        assert np.array_equal(xn, O.residual_bf16(xb, Yh)), l
        if l in (0, 11, 23):
            x = O.bf16_to_f64(xb)
            y = np.zeros(2048)
            for j in range(8):
                deq = [O.dequantize(*O.ternarize_absmean(m)) for m in _raw_expert(cfg, l, int(ridx[0, j]))]
                y += rw[0, j] * O.expert_ffn(x, *deq)[3][0]
            err = O.max_normalized_error(Yh, y[None])
            say(f"  one-token stack layer {l}: max normalized error {err:.2e}")
            assert err <= TOL
        xb = xn
    final = host(xs[L]).copy()
    idx_eager = host(idx).copy()

    # the whole chain as one graph (in place on one residual buffer), replayed
    Xw = torch.empty((1, 2048), dtype=torch.int16, device="cuda")
    idx_g = torch.zeros_like(idx)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.capture_begin()
        for l in range(L):
            tm.moe_forward(Ws[l], xs[0] if l == 0 else Xw, None, ws, idx=idx_g[l], resid_out=Xw)
        g.capture_end()
    torch.cuda.synchronize()
    for rep in range(3):
        Xw.fill_(0)
        idx_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(host(Xw), final), rep
        assert np.array_equal(host(idx_g), idx_eager), rep


@pytest.mark.parametrize("cfg,T,bias_kind", [(2, 1, None), (2, 3, None), (3, 64, "zipf")])
def test_layer_experts_on_host(tm, layers, cfg, T, bias_kind):
    """Experts in pinned host memory that the kernels read over PCIe (the
    streaming variant): the oracle's top-8 and Y, and the device-resident
    layer's result bit for bit (the same kernels run on the same bytes);
    for one token, a captured graph replays it identically."""
    say(f"layer with host-resident experts cfg={cfg} T={T}")
    W = layers(cfg, 0, bias_kind)
    Wh = tm.experts_on_host(W)
    xb = ti.activations(cfg, T)
    got = _run_layer(tm, Wh, xb)
    on_dev = _run_layer(tm, W, xb)
    for key in ("Y", "idx", "w", "pos"):
        assert np.array_equal(got[key], on_dev[key]), key
    ref = O.moe_layer(xb, ti.router_matrix(cfg, 0), ti.router_bias(cfg, bias_kind),
                      lambda e: _raw_expert(cfg, 0, e), k=8)
    assert np.array_equal(got["idx"], ref["idx"])
    err = O.max_normalized_error(got["Y"], ref["Y"])
    say(f"  Y max normalized error {err:.2e}")
    assert err <= TOL
    if T == 1:
        X = bf16_dev(xb)
        Y = torch.zeros((1, 2048), dtype=torch.float32, device="cuda")
        ws = ws_bytes(tm.moe_workspace_bytes(1, Wh))
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g.capture_begin()
            tm.moe_forward(Wh, X, Y, ws)
            g.capture_end()
        torch.cuda.synchronize()
        for rep in range(3):
            Y.zero_()
            torch.cuda.synchronize()
            g.replay()
            assert np.array_equal(host(Y), got["Y"]), rep


# ------------------------------------------------------------ attention half
_ATTN_DENSE = {}


def _attn_dense(cfg, layer):
    if (cfg, layer) not in _ATTN_DENSE:
        dq = O.dequantize(*O.ternarize_absmean(ti.attn_qkv_matrix(cfg, layer)))
        do = O.dequantize(*O.ternarize_absmean(ti.attn_o_matrix(cfg, layer)))
        _ATTN_DENSE[(cfg, layer)] = (dq[:2048], dq[2048:2560], dq[2560:], do)
    return _ATTN_DENSE[(cfg, layer)]


@pytest.mark.parametrize("layer,P,chunk", [(0, 37, 37), (3, 37, 37), (1, 700, 50), (7, 700, 650), (2, 530, 1)])
def test_attention_parity(tm, layer, P, chunk):
    """The attention half over a P-token sequence, fed in chunks (prefill, then
    one-token decode steps for chunk 1) through the cache, against the
    oracle over the whole sequence: O per position within tolerance, the
    residual bit for bit from O. Sliding caches take the smallest allowed
    capacity (window + chunk - 1), so positions wrap around the ring."""
    from oracle import attention_oracle as AO
    from ternary_weight_moe_base_amd import synthetic

    cfg = 5
    glob = AO.is_global_layer(layer)
    say(f"attention layer={layer} ({'global' if glob else 'sliding'}) P={P} chunk={chunk}")
    W = synthetic.build_attention(cfg, layer, glob)
    cap = P if glob else 512 + chunk - 1
    kc, vc = tm.kv_cache(W, cap)
    xb = ti.activations(cfg, P + 3)[3:]
    X = bf16_dev(xb)
    Ob = torch.empty((P, 2048), dtype=torch.float32, device="cuda")
    Xo = torch.empty((P, 2048), dtype=torch.int16, device="cuda")
    ws = ws_bytes(tm.attention_workspace_bytes(chunk, W))
    for p0 in range(0, P, chunk):
        T = min(chunk, P - p0)
        tm.attention_forward(W, X[p0:p0 + T], p0, kc, vc, ws, O=Ob[p0:p0 + T], X_out=Xo[p0:p0 + T])
    got_o, got_x = host(Ob), host(Xo).view(np.uint16)
    ref = AO.attention_half(xb, *_attn_dense(cfg, layer), glob)
    err = O.max_normalized_error(got_o, ref["o"])
    say(f"  O max normalized error {err:.2e}")
    assert err <= TOL
    assert np.array_equal(got_x, O.residual_bf16(xb, got_o))


def test_attention_decode_graph_replay(tm):
    """One-token attention steps captured in a HIP graph (positions advance
    through the cache between replays) equal the eager steps bit for bit."""
    from ternary_weight_moe_base_amd import synthetic

    W = synthetic.build_attention(5, 0, False)
    xb = ti.activations(5, 12)
    X = bf16_dev(xb)
    outs = []
    for graph in (False, True):
        kc, vc = tm.kv_cache(W, 519)  # window + 8 - 1: the 8-token prefill below
        ws = ws_bytes(tm.attention_workspace_bytes(1, W))
        O_ = torch.zeros((1, 2048), dtype=torch.float32, device="cuda")
        tm.attention_forward(W, X[:8], 0, kc, vc, ws_bytes(tm.attention_workspace_bytes(8, W)), O=torch.empty((8, 2048), dtype=torch.float32, device="cuda"))
        res = []
        for p in range(8, 12):
            if graph:
                g = torch.cuda.CUDAGraph()
                s_ = torch.cuda.Stream()
                s_.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s_):
                    g.capture_begin()
                    tm.attention_forward(W, X[p:p + 1], p, kc, vc, ws, O=O_)
                    g.capture_end()
                torch.cuda.synchronize()
                g.replay()
            else:
                tm.attention_forward(W, X[p:p + 1], p, kc, vc, ws, O=O_)
            res.append(host(O_).copy())
        outs.append(res)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


# -------------------------------------------------------------------- LM head
def _lm_head(tm, xb, Wd, k, with_logits=True):
    T = xb.shape[0]
    V = Wd.shape[0]
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    val = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, V), dtype=torch.float32, device="cuda") if with_logits else None
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ws_bytes(tm.lm_head_workspace_bytes(T, V, k))
    tm.lm_head_topk(bf16_dev(xb), Wd, k, idx, val, ws, logits=lg, n_fixup=nf)
    return host(idx), host(val), (host(lg) if with_logits else None), int(host(nf)[0])


@pytest.mark.parametrize("T,H,V,k", [(1, 2048, 3000, 8), (2, 512, 1537, 16), (4, 1024, 2049, 1), (1, 4096, 777, 5),
                                     (4, 2048, 5000, 16), (1, 512, 17, 16)])
def test_lm_head_parity(tm, T, H, V, k):
    say(f"lm head T={T} H={H} V={V} k={k}")
    g = np.random.default_rng(T * 1000 + V)
    xb = ti.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    Wb = ti.f32_to_bf16_bits((g.standard_normal((V, H)) * 0.02).astype(np.float32))
    idx, val, lg, nfix = _lm_head(tm, xb, dev(Wb.view(np.int16)), k)
    ridx, rval, rL, _ = O.lm_head_topk(xb, Wb, k)
    assert nfix == 0
    assert np.array_equal(idx, ridx)
    assert O.max_normalized_error(val, rval) <= TOL
    assert O.max_normalized_error(lg, rL) <= TOL


def test_lm_head_exact_ties_and_near_ties(tm):
    # rows 700 and 1200 duplicate row 40 (exact ties: ids ascending, no
    # recompute); then row 1500 differs from row 40 only where x is 2^-60, so
    # its logit is larger by far less than a float64 ulp: only the
    # double-double path ranks it first
    H, V, k = 512, 2000, 4
    g = np.random.default_rng(77)
    x = g.standard_normal((1, H)).astype(np.float32)
    x[0, 5] = 2.0 ** -60
    xb = ti.f32_to_bf16_bits(x)
    W = (g.standard_normal((V, H)) * 0.02).astype(np.float32)
    W[40] = np.sign(x[0]) * 0.05  # the largest logit by far
    W[40, 5] = 0.03125
    Wb = ti.f32_to_bf16_bits(W)
    Wb[700] = Wb[40]
    Wb[1200] = Wb[40]
    idx, val, _, nfix = _lm_head(tm, xb, dev(Wb.view(np.int16)), k, with_logits=False)
    ridx, _, _, _ = O.lm_head_topk(xb, Wb, k)
    assert nfix == 0
    assert np.array_equal(idx, ridx) and idx[0, :3].tolist() == [40, 700, 1200]
    Wb[1500] = Wb[40]
    Wb[1500, 5] += 1  # one bf16 ulp more (positive value)
    idx, val, _, nfix = _lm_head(tm, xb, dev(Wb.view(np.int16)), k, with_logits=False)
    ridx, _, _, n_exact = O.lm_head_topk(xb, Wb, k)
    assert n_exact == 1 and nfix == 1
    assert np.array_equal(idx, ridx) and idx[0].tolist() == [1500, 40, 700, 1200]


def test_lm_head_full_vocabulary(tm):
    # the model's head: 151,936 x 2048 bf16 (622 MB), one token, k = 16; the
    # device-drawn table equals the host draw on sampled rows, and the top-16
    # and all logits match the oracle over the whole vocabulary
    from ternary_weight_moe_base_amd import synthetic
    cfg, V, H, k = 5, ti.VOCAB, 2048, 16
    Wd = synthetic.lm_head_table(cfg)
    for v0 in (0, 77777, V - 3):
        assert np.array_equal(host(Wd[v0:v0 + 3]).view(np.uint16), ti.lm_head_rows(cfg, v0, v0 + 3))
    xb = ti.activations(cfg, 1)
    idx, val, lg, nfix = _lm_head(tm, xb, Wd, k)
    say("  drawing the table on the host for the oracle")
    Wh = np.concatenate([ti.lm_head_rows(cfg, v0, min(v0 + 16384, V)) for v0 in range(0, V, 16384)])
    ridx, rval, rL, _ = O.lm_head_topk(xb, Wh, k)
    assert nfix == 0
    assert np.array_equal(idx, ridx)
    assert O.max_normalized_error(val, rval) <= TOL
    assert O.max_normalized_error(lg, rL) <= TOL
    say(f"  top-{k} ids {idx[0].tolist()}")


# ------------------------------------------------------------- native driver
@pytest.mark.parametrize("args", [["layer", "--tokens", "1", "--layers", "2", "--steps", "20", "--warmup", "2"],
                                  ["layer", "--tokens", "64", "--layers", "1", "--steps", "5", "--warmup", "1"],
                                  ["layer", "--tokens", "1", "--layers", "1", "--steps", "5", "--warmup", "1",
                                   "--host-experts", "1"],
                                  ["lmhead", "--vocab", "20000", "--steps", "5", "--warmup", "1"],
                                  ["copy", "--mib", "64", "--steps", "3"]])
def test_native_driver_runs(args):
    """The C-ABI driven with no Python in the process: the native driver builds
    its synthetic model through the library and runs each workload."""
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.dirname(__file__)), "ternary_weight_moe_base_amd", "tmoe_run")
    say(f"tmoe_run {' '.join(args)}")
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr
    assert ("us/step" in r.stdout) or ("GB/s" in r.stdout), r.stdout


def test_native_driver_issue_costs():
    """The issue-cost calibration of the native driver: every instruction kind
    gets a positive cost per wavefront instruction, a product costs more than any
    vector instruction, and the clock line is printed."""
    import re
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.dirname(__file__)), "ternary_weight_moe_base_amd", "tmoe_run")
    say("tmoe_run issue")
    r = subprocess.run([exe, "issue"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    rows = dict()
    for line in r.stdout.splitlines():
        m = re.match(r"\s+(v_\w+)\s+([0-9.]+)\s+([0-9.]+)\s*$", line)
        if m:
            rows[m.group(1)] = (float(m.group(2)), float(m.group(3)))
    assert len(rows) == 10, r.stdout
    assert all(a > 0 and b > 0 for a, b in rows.values())
    mfma = rows["v_mfma_f32_16x16x32_bf16"][1]
    assert all(mfma > b for k, (a, b) in rows.items() if not k.startswith("v_mfma"))
    assert "core clock" in r.stdout
