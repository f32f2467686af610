"""C ABI checks that need no GPU: every declared symbol is exported, the host
weight steps match the oracle bit for bit, and argument errors come back as
documented status codes before anything touches HIP."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
import tmoe_inputs as ti

tm = pytest.importorskip("ternary_weight_moe_base_amd")
lib = tm.lib
HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tmoe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tmoe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 24
    for n in names:
        assert hasattr(lib, n), n
        assert n in tm._abi.SIGNATURES, f"{n} not bound in the Python binding"


def test_status_strings():
    for code, name in tm._abi._NAMES.items():
        assert tm.status_str(code) == name
    assert tm.status_str(-99) == "TMOE_E_UNKNOWN"
    assert tm.version() == 100


@pytest.mark.parametrize("R,K", [(1, 1), (3, 7), (9, 23), (33, 517), (16, 2048), (64, 512)])
def test_host_ternarize_pack_match_oracle(R, K):
    g = np.random.default_rng(R * 1000 + K)
    W = g.standard_normal((R, K)).astype(np.float32)
    W[0, : min(K, 3)] = 0.0
    T, s = tm.ternarize_absmean_host(W)
    To, so = O.ternarize_absmean(W)
    assert np.array_equal(T, To) and np.array_equal(s, so)
    P = tm.pack_host(T, ldp=(K + 4) // 5 + 5)
    assert np.array_equal(P[:, : (K + 4) // 5], O.pack_trits(To))
    assert np.array_equal(tm.unpack_host(P, K), To)
    assert tm.validate_packed_host(P[:, : (K + 4) // 5], K) == 0


def test_host_synthetic_weights_match_oracle():
    W = ti.expert_matrix(2, 0, 7, ti.MAT_DOWN)
    T, s = tm.ternarize_absmean_host(W)
    To, so = O.ternarize_absmean(W)
    assert np.array_equal(T, To) and np.array_equal(s, so)


def test_host_scale_sums_in_index_order():
    # |w| = (1, 2^-53, 2^-24, 2^-53): index order rounds the mean to 0.25, a
    # pairwise order would give 0.25 + 2^-25 (see the device test of the same rows)
    base = np.array([1.0, 2.0 ** -53, 2.0 ** -24, 2.0 ** -53])
    W = np.stack([base, 4.0 * base, -0.5 * base]).astype(np.float32)
    T, s = tm.ternarize_absmean_host(W)
    assert np.array_equal(s, np.array([0.25, 1.0, 0.125], np.float32))
    t_ref, s_ref = O.ternarize_absmean(W)
    assert np.array_equal(s, s_ref) and np.array_equal(T, t_ref)


def test_host_exhaustive_codes():
    import itertools
    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=5)), dtype=np.int8)
    P = tm.pack_host(tuples)
    assert np.array_equal(P, O.pack_trits(tuples))


def test_host_errors():
    i8 = ctypes.c_void_p
    assert lib.tmoe_ternarize_absmean_host(None, 2, 3, None, None) == tm._abi.TMOE_E_ARG
    assert lib.tmoe_ternarize_absmean_host(None, -1, 3, None, None) == tm._abi.TMOE_E_ARG
    assert "null" in lib.tmoe_last_error().decode() or "negative" in lib.tmoe_last_error().decode()
    W = np.array([[1.0, np.nan]], np.float32)
    with pytest.raises(tm.TmoeError) as ei:
        tm.ternarize_absmean_host(W)
    assert ei.value.status == tm._abi.TMOE_E_ARG
    with pytest.raises(tm.TmoeError) as ei:
        tm.pack_host(np.array([[2, 0]], np.int8))
    assert ei.value.status == tm._abi.TMOE_E_ARG
    T = np.zeros((2, 11), np.int8)
    rc = lib.tmoe_pack_host(T.ctypes.data_as(i8), 2, 11, None, 2)  # ldp < ceil(11/5)
    assert rc == tm._abi.TMOE_E_SHAPE
    bad = np.array([[0, 243, 7], [255, 1, 2]], np.uint8)
    with pytest.raises(tm.TmoeError) as ei:
        tm.validate_packed_host(bad, 15)
    assert ei.value.status == tm._abi.TMOE_E_BADPACK
    with pytest.raises(tm.TmoeError) as ei:
        tm.unpack_host(bad, 15)
    assert ei.value.status == tm._abi.TMOE_E_BADPACK
    # empty inputs are fine
    assert lib.tmoe_ternarize_absmean_host(None, 0, 5, None, None) == 0
    assert lib.tmoe_pack_host(None, 0, 5, None, 1) == 0


def test_tiled_bytes_formula():
    for R, K in [(1, 1), (16, 2048), (512, 2048), (2048, 512), (17, 23), (100, 517)]:
        Kb = (K + 4) // 5
        Q = max(2, math.ceil(Kb / 4))
        Q += Q & 1
        assert tm.tiled_bytes(R, K) == math.ceil(R / 16) * 64 * Q
    # about 1.5% (gate/up) and 1% (down) above the canonical bytes
    assert tm.tiled_bytes(512, 2048) / (512 * 410) < 1.016
    assert tm.tiled_bytes(2048, 512) / (2048 * 103) < 1.011
    assert tm.tiled_bytes(0, 5) == 0


def test_device_entry_points_reject_bad_arguments_without_gpu():
    E = tm._abi
    # null / misaligned pointers and small workspaces return before any HIP call
    assert lib.tmoe_ternary_linear(None, None, None, 4, 8, None, 8, 2, None, 4, None, 0) == E.TMOE_E_ARG
    assert lib.tmoe_ternary_linear(None, 16, 16, 4, 8, 16, 4, 2, 16, 4, None, 0) == E.TMOE_E_SHAPE  # ldx < K
    assert lib.tmoe_ternary_linear(None, 17, 16, 4, 8, 16, 8, 2, 16, 4, 16, 1 << 20) == E.TMOE_E_ALIGN
    assert lib.tmoe_linear_workspace_bytes(2, 8) == 0  # the linear kernels need no scratch memory
    assert lib.tmoe_ternary_linear(None, None, None, 0, 8, None, 8, 2, None, 0, None, 0) == E.TMOE_OK  # N = 0
    assert lib.tmoe_router_topk(None, 16, 4, 2048, 16, None, 256, 0, 16, 16, None, None, 16, 1 << 20) == E.TMOE_E_SHAPE
    assert lib.tmoe_router_topk(None, 16, 4, 2048, 16, None, 2048, 8, 16, 16, None, None, 16, 1 << 20) == E.TMOE_E_UNSUPPORTED
    assert lib.tmoe_router_topk(None, 16, 4, 2048, 16, None, 256, 8, 16, 16, None, None, 16, 16) == E.TMOE_E_WORKSPACE
    assert lib.tmoe_router_topk(None, 16, 0, 2048, 16, None, 256, 8, 16, 16, None, None, None, 0) == E.TMOE_OK
    assert lib.tmoe_group_by_expert(None, None, 4, 8, 256, None, None, None, None, None, None, 0) == E.TMOE_E_ARG
    assert lib.tmoe_combine(None, None, None, None, 1, 8, 2048, None, None, None) == E.TMOE_E_ARG
    assert lib.tmoe_combine(None, 16, 16, 16, 1, 8, 2048, 16, None, 16) == E.TMOE_E_ARG  # resid_out w/o resid_in
    assert lib.tmoe_synth_ih12(None, 1, 0, 1, 0, -1, 1.0, 16) == E.TMOE_E_ARG
    assert lib.tmoe_repack_tiled(None, 16, 4, 23, 4, 16) == E.TMOE_E_SHAPE  # ldp < ceil(23/5)
    # the canonical-byte linear: the tiled image (256-byte aligned) plus the linear's own scratch
    for N, K, T in [(512, 2048, 4), (17, 23, 3), (300, 1000, 37)]:
        need = lib.tmoe_linear_packed_workspace_bytes(N, K, T)
        assert need == math.ceil(tm.tiled_bytes(N, K) / 256) * 256 + lib.tmoe_linear_workspace_bytes(T, K)
    assert lib.tmoe_linear_packed_workspace_bytes(0, 8, 4) == 0
    f = lib.tmoe_ternary_linear_packed
    assert f(None, 16, 1, 16, 4, 8, 16, 8, 2, 16, 4, 16, 1 << 20) == E.TMOE_E_SHAPE  # ldp < ceil(8/5)
    assert f(None, 16, 2, 16, 4, 8, 16, 4, 2, 16, 4, 16, 1 << 20) == E.TMOE_E_SHAPE  # ldx < K
    assert f(None, None, 2, None, 4, 8, None, 8, 2, None, 4, 16, 1 << 20) == E.TMOE_E_ARG
    assert f(None, 16, 2, 16, 4, 8, 16, 8, 2, 16, 4, 16, 16) == E.TMOE_E_WORKSPACE
    assert f(None, 16, 2, 16, 4, 8, 16, 8, 2, 16, 4, 17, 1 << 20) == E.TMOE_E_WORKSPACE  # misaligned ws
    assert f(None, None, 2, None, 0, 8, None, 8, 2, None, 0, None, 0) == E.TMOE_OK  # N = 0


def test_lm_head_rejects_bad_arguments_without_gpu():
    E = tm._abi
    V, k = 151936, 16
    ws = tm.lm_head_workspace_bytes(1, V, k)
    assert ws >= V * 8  # the float64 logits of every token id
    f = lib.tmoe_lm_head_topk
    assert f(None, None, 1, 2048, 16, V, k, 16, 16, None, None, 16, ws) == E.TMOE_E_ARG
    assert f(None, 16, 3, 2048, 16, V, k, 16, 16, None, None, 16, ws) == E.TMOE_E_UNSUPPORTED  # T = 3
    assert f(None, 16, 1, 3000, 16, V, k, 16, 16, None, None, 16, ws) == E.TMOE_E_UNSUPPORTED  # H
    assert f(None, 16, 1, 2048, 16, V, 17, 16, 16, None, None, 16, ws) == E.TMOE_E_UNSUPPORTED  # k > 16
    assert f(None, 16, 1, 2048, 16, 8, 8, 16, 16, None, None, 16, ws) == E.TMOE_E_SHAPE  # k >= V
    assert f(None, 16, 1, 2048, 16, (1 << 20) + 1, k, 16, 16, None, None, 16, ws) == E.TMOE_E_UNSUPPORTED  # V too large
    assert f(None, 18, 1, 2048, 16, V, k, 16, 16, None, None, 16, ws) == E.TMOE_E_ALIGN
    assert f(None, 16, 1, 2048, 16, V, k, 16, 16, None, None, 16, ws - 1) == E.TMOE_E_WORKSPACE
    assert f(None, 16, 0, 2048, 16, V, k, 16, 16, None, None, None, 0) == E.TMOE_OK  # T = 0


def test_layer_struct_validation_without_gpu():
    Ew = tm._abi
    s = tm._abi.MoEWeightsStruct()
    s.hidden, s.inter, s.n_experts, s.top_k = 2048, 512, 256, 8
    out = ctypes.c_size_t(0)
    assert lib.tmoe_moe_workspace_bytes(4, ctypes.byref(s), ctypes.byref(out)) == Ew.TMOE_E_ARG  # null weights
    for name in ("gate_p", "up_p", "down_p", "gate_s", "up_s", "down_s", "router_w"):
        setattr(s, name, 256)
    s.stride_gu, s.stride_d = tm.tiled_bytes(512, 2048), tm.tiled_bytes(2048, 512)
    assert lib.tmoe_moe_workspace_bytes(4, ctypes.byref(s), ctypes.byref(out)) == 0
    assert out.value > 4 * 8 * 512 * 4  # fp32 h of every (token, slot) pair
    assert lib.tmoe_moe_workspace_bytes(64, ctypes.byref(s), ctypes.byref(out)) == 0
    assert out.value > 64 * 8 * 2048 * 4  # batched path: expert outputs before the combine
    s.stride_gu -= 16
    assert lib.tmoe_moe_workspace_bytes(4, ctypes.byref(s), ctypes.byref(out)) == Ew.TMOE_E_SHAPE
    s.stride_gu += 16
    s.top_k = 17
    assert lib.tmoe_moe_workspace_bytes(4, ctypes.byref(s), ctypes.byref(out)) == Ew.TMOE_E_SHAPE
    s.top_k = 8
    s.reserved = 1
    assert lib.tmoe_moe_workspace_bytes(4, ctypes.byref(s), ctypes.byref(out)) == Ew.TMOE_E_ARG
    s.reserved = 0
    assert lib.tmoe_moe_forward(None, ctypes.byref(s), None, 4, None, None, None, 0) == Ew.TMOE_E_ARG
    assert lib.tmoe_moe_forward(None, ctypes.byref(s), None, 0, None, None, None, 0) == Ew.TMOE_OK


def test_native_driver_rejects_bad_arguments_without_gpu():
    """The native driver (built next to the library) parses and checks its
    arguments before it touches HIP, so this runs on a machine with no GPU."""
    import subprocess

    exe = os.path.join(os.path.dirname(tm.__file__), "tmoe_run")
    assert os.access(exe, os.X_OK), "tmoe_run is built by ternary_weight_moe_base_amd.build"
    for args, msg in ((["layer", "--tokens", "0"], "out of range"), (["layer", "--bogus", "1"], "unknown option"),
                      (["layer", "--steps"], "missing value"), (["layer", "--layers", "65"], "out of range")):
        r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=60)
        assert r.returncode == 1 and msg in r.stderr, (args, r.returncode, r.stderr)


def test_host_alloc_rejects_bad_arguments_without_gpu():
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.tmoe_host_alloc(0, ctypes.byref(h), ctypes.byref(d)) == -1  # TMOE_E_ARG
    assert lib.tmoe_host_alloc(64, None, ctypes.byref(d)) == -1
    assert lib.tmoe_host_alloc(64, ctypes.byref(h), None) == -1
    assert lib.tmoe_host_free(None) == 0


def test_attention_rejects_bad_arguments_without_gpu():
    """Shape and cache checks return status codes before anything touches HIP
    (the pointers are aligned stand-ins that are never dereferenced)."""
    W = tm._abi.AttnWeightsStruct()
    W.hidden, W.n_heads, W.n_kv_heads, W.head_dim, W.rotary_dim, W.window, W.reserved = 2048, 16, 4, 128, 64, 512, 0
    W.rope_base = 10000.0
    W.qkv_p = W.qkv_s = W.o_p = W.o_s = 1 << 20
    fake = ctypes.c_void_p(1 << 21)
    ws_n = lib.tmoe_attention_workspace_bytes(1, ctypes.byref(W))
    assert ws_n > 0
    call = lambda W_, T, pos0, cap: lib.tmoe_attention_forward(None, ctypes.byref(W_), fake, T, pos0, fake, fake, cap,
                                                               fake, None, fake, ws_n * 64)
    assert call(W, 0, 0, 512) == 0  # nothing to do
    assert call(W, 4, 0, 514) == -2  # sliding: capacity < window + T - 1
    W.window = 0
    assert call(W, 4, 100, 103) == -2  # global: capacity < pos0 + T
    W.n_kv_heads = 8
    assert call(W, 1, 0, 4096) == -6  # head shape outside the built kernels
    assert lib.tmoe_attention_workspace_bytes(1, ctypes.byref(W)) == 0
    W.n_kv_heads, W.reserved = 4, 1
    assert call(W, 1, 0, 4096) == -1
