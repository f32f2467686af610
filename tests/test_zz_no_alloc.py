"""The allocation-free layer call (tmoe_moe_forward_noalloc, scratch in the
library's fixed per-GPU array) against the workspace layer call
(tmoe_moe_forward) on the same inputs, through the C ABI: calls in a row with
shrinking token counts (each call finds the previous call's data in the
array), both layer paths (batched and one-token decode) and both clamp
modes; results must be bit-identical, since the same kernels run."""
import math

import numpy as np
import pytest

import tmoe_inputs as ti

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _outputs(T, k):
    Y = torch.full((T, 2048), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    pos = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    return Y, idx, w, pos


def test_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_moe_base_amd as tm
    from ternary_weight_moe_base_amd import synthetic

    W = synthetic.build_layer(3, 0, "zipf")
    k = W.top_k
    for T, clamp in ((256, 7.0), (64, math.inf), (5, 7.0), (1, 7.0), (1, math.inf)):
        say(f"no-alloc layer T={T} clamp={clamp}")
        X = synthetic.activations(3, T, layer=T)
        ref = _outputs(T, k)
        ws = torch.full((tm.moe_workspace_bytes(T, W),), 255, dtype=torch.uint8, device="cuda")
        tm.moe_forward(W, X, ref[0], ws, clamp=clamp, idx=ref[1], w=ref[2], pos=ref[3])
        got = _outputs(T, k)
        tm.moe_forward_noalloc(W, X, got[0], clamp=clamp, idx=got[1], w=got[2], pos=got[3])
        torch.cuda.synchronize()
        for name, a, b in zip(("Y", "idx", "w", "pos"), ref, got):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
        assert not torch.isnan(got[0]).any()
    # the residual stream (the 24-layer stack's form) through the same array
    X = synthetic.activations(3, 3, layer=7)
    Xr_ref, Xr = torch.empty_like(X), torch.empty_like(X)
    ws = torch.zeros(tm.moe_workspace_bytes(3, W), dtype=torch.uint8, device="cuda")
    tm.moe_forward(W, X, None, ws, resid_out=Xr_ref)
    tm.moe_forward_noalloc(W, X, None, resid_out=Xr)
    torch.cuda.synchronize()
    assert torch.equal(Xr, Xr_ref)


def test_noalloc_rejects_requests_beyond_the_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_moe_base_amd as tm
    from ternary_weight_moe_base_amd import synthetic

    W = synthetic.build_layer(2, 0, None, experts=16)
    T = 1
    while tm.moe_workspace_bytes(T, W) <= tm.NOALLOC_SCRATCH_BYTES:
        T *= 2
    say(f"no-alloc layer T={T}: workspace {tm.moe_workspace_bytes(T, W)} bytes > the array")
    X = synthetic.activations(2, T)
    Y = torch.full((T, 2048), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(tm.TmoeError) as e:
        tm.moe_forward_noalloc(W, X, Y)
    assert e.value.status == tm._abi.TMOE_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(Y).all()  # nothing was enqueued
    # the largest request that fits still runs, and matches the workspace call
    while tm.moe_workspace_bytes(T, W) > tm.NOALLOC_SCRATCH_BYTES:
        T -= max(1, T // 64)
    say(f"no-alloc layer T={T}: the largest that fits, {tm.moe_workspace_bytes(T, W)} bytes")
    X = synthetic.activations(2, T)
    Y, Y_ref = (torch.empty((T, 2048), dtype=torch.float32, device="cuda") for _ in range(2))
    tm.moe_forward_noalloc(W, X, Y)
    ws = torch.zeros(tm.moe_workspace_bytes(T, W), dtype=torch.uint8, device="cuda")
    tm.moe_forward(W, X, Y_ref, ws)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref)
