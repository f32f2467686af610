"""Python binding of libtmoe, the ternary Mixture-of-Experts expert layer for
MI355X (gfx950).

Argument marshalling only: every function here forwards to the C ABI declared
in ``include/tmoe.h`` (same names without the ``tmoe_`` prefix). Device
buffers are PyTorch tensors on the GPU (``data_ptr()``), launched on
``torch.cuda.current_stream()``; host buffers are NumPy arrays. There is no
CPU fallback: importing this package fails if ``libtmoe.so`` is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _abi

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtmoe.so")


class TmoeError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {_abi.status_name(status)} ({status}): {message}")
        self.status = status


_lib = None


def _load() -> ctypes.CDLL:
    """Loads libtmoe.so on first use; raises ImportError when it is not built
    (there is no fallback implementation)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} not built; run `python -m ternary_weight_moe_base_amd.build`")
        # PyTorch first: its HIP runtime (soname libamdhip64.so.7) is then the one
        # libtmoe.so binds to. Loaded the other way round, the process holds two
        # HIP runtimes, and the second to initialise finds no device.
        import torch  # noqa: F401
        lib = ctypes.CDLL(_LIB_PATH)
        _abi.declare(lib)
        _abi.bind_status(lib)
        _lib = lib
    return _lib


def __getattr__(name):
    if name == "lib":
        return _load()
    raise AttributeError(name)

LAYOUT_HIDDEN = 2048
LAYOUT_INTER = 512


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise TmoeError(rc, where, _load().tmoe_last_error().decode())


def status_str(code: int) -> str:
    return _load().tmoe_status_str(code).decode()


def version() -> int:
    return _load().tmoe_version()


# ------------------------------------------------------------------ helpers
def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (None for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    return t.data_ptr()


def _np(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream=None) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# --------------------------------------------------------- host weight steps
def ternarize_absmean_host(W: np.ndarray):
    """fp32 [R][K] -> (int8 trits [R][K], fp32 scales [R])."""
    W, pw = _np(W, np.float32)
    R, K = W.shape
    T = np.empty((R, K), np.int8)
    s = np.empty(R, np.float32)
    _check(_load().tmoe_ternarize_absmean_host(pw, R, K, T.ctypes.data_as(ctypes.c_void_p),
                                           s.ctypes.data_as(ctypes.c_void_p)), "ternarize_absmean_host")
    return T, s


def pack_host(T: np.ndarray, ldp: int | None = None) -> np.ndarray:
    T, pt = _np(T, np.int8)
    R, K = T.shape
    ldp = (K + 4) // 5 if ldp is None else ldp
    P = np.zeros((R, ldp), np.uint8)
    _check(_load().tmoe_pack_host(pt, R, K, P.ctypes.data_as(ctypes.c_void_p), ldp), "pack_host")
    return P


def unpack_host(P: np.ndarray, K: int) -> np.ndarray:
    P, pp = _np(P, np.uint8)
    R, ldp = P.shape
    T = np.empty((R, K), np.int8)
    _check(_load().tmoe_unpack_host(pp, R, K, ldp, T.ctypes.data_as(ctypes.c_void_p)), "unpack_host")
    return T


def validate_packed_host(P: np.ndarray, K: int) -> int:
    """Number of invalid bytes (> 242); raises TmoeError(TMOE_E_BADPACK) if any."""
    P, pp = _np(P, np.uint8)
    R, ldp = P.shape
    n = ctypes.c_int64(0)
    rc = _load().tmoe_validate_packed_host(pp, R, K, ldp, ctypes.byref(n))
    if rc not in (0, _abi.TMOE_E_BADPACK):
        _check(rc, "validate_packed_host")
    if rc:
        raise TmoeError(rc, "validate_packed_host", f"{n.value} invalid bytes")
    return n.value


def tiled_bytes(R: int, K: int) -> int:
    return _load().tmoe_tiled_bytes(R, K)


# ------------------------------------------------------- device weight steps
def synth_ih12(out, stream_id: int, first: int = 0, key0: int = 0x7E4A, key1: int = 0, mult: float = 1.0,
               stream=None) -> None:
    """Fills the fp32 tensor `out` with Irwin-Hall(12) draws of Philox4x64-10 stream `stream_id`."""
    _check(_load().tmoe_synth_ih12(_stream(stream), key0, key1, stream_id, first, out.numel(), mult, _ptr(out)),
           "synth_ih12")


def ternarize_pack(W, P, s, stream=None) -> None:
    """W fp32 [R][K] -> canonical P uint8 [R][ldp], scales s fp32 [R] (device)."""
    R, K = W.shape
    _check(_load().tmoe_ternarize_pack(_stream(stream), _ptr(W), R, K, _ptr(P), P.shape[1], _ptr(s)), "ternarize_pack")


def unpack(P, K: int, T, stream=None) -> None:
    R, ldp = P.shape
    _check(_load().tmoe_unpack(_stream(stream), _ptr(P), R, K, ldp, _ptr(T)), "unpack")


def repack_tiled(P, K: int, Pt, stream=None) -> None:
    R, ldp = P.shape
    _check(_load().tmoe_repack_tiled(_stream(stream), _ptr(P), R, K, ldp, _ptr(Pt)), "repack_tiled")


def unpack_tiled(Pt, R: int, K: int, T, stream=None) -> None:
    _check(_load().tmoe_unpack_tiled(_stream(stream), _ptr(Pt), R, K, _ptr(T)), "unpack_tiled")


# ------------------------------------------------------------ ternary linear
def linear_workspace_bytes(T: int, K: int) -> int:
    return _load().tmoe_linear_workspace_bytes(T, K)


def ternary_linear(Pt, s, N: int, K: int, X, Y, ws, stream=None) -> None:
    """Y[T][N] fp32 = s * (trits @ X^T); X bf16 bits (int16/uint16 tensor) [T][ldx]."""
    T, ldx = X.shape
    _check(_load().tmoe_ternary_linear(_stream(stream), _ptr(Pt), _ptr(s), N, K, _ptr(X), ldx, T, _ptr(Y), Y.shape[1],
                                   _ptr(ws), ws.numel() * ws.element_size()), "ternary_linear")


def linear_packed_workspace_bytes(N: int, K: int, T: int) -> int:
    return _load().tmoe_linear_packed_workspace_bytes(N, K, T)


def ternary_linear_packed(P, s, K: int, X, Y, ws, stream=None) -> None:
    """The same product from canonical packed bytes P uint8 [N][ldp] (repacked into ws first)."""
    N, ldp = P.shape
    T, ldx = X.shape
    _check(_load().tmoe_ternary_linear_packed(_stream(stream), _ptr(P), ldp, _ptr(s), N, K, _ptr(X), ldx, T, _ptr(Y),
                                          Y.shape[1], _ptr(ws), ws.numel() * ws.element_size()), "ternary_linear_packed")


# -------------------------------------------------------------------- router
def router_workspace_bytes(T: int, E: int) -> int:
    return _load().tmoe_router_workspace_bytes(T, E)


def router_topk(X, Wr, bias, k: int, idx, w, ws, logits=None, n_fixup=None, stream=None) -> None:
    T, H = X.shape
    E = Wr.shape[0]
    _check(_load().tmoe_router_topk(_stream(stream), _ptr(X), T, H, _ptr(Wr), _ptr(bias), E, k, _ptr(idx), _ptr(w),
                                _ptr(logits), _ptr(n_fixup), _ptr(ws), ws.numel() * ws.element_size()),
           "router_topk")


# ------------------------------------------------------------------- LM head
def lm_head_workspace_bytes(T: int, V: int, k: int) -> int:
    return _load().tmoe_lm_head_workspace_bytes(T, V, k)


def lm_head_topk(X, W, k: int, idx, val, ws, logits=None, n_fixup=None, stream=None) -> None:
    """Logits of the bf16 output table W [V][H] for X [T][H] (bf16 bit patterns)
    and the certified top-k token ids / logits."""
    T, H = X.shape
    V = W.shape[0]
    _check(_load().tmoe_lm_head_topk(_stream(stream), _ptr(X), T, H, _ptr(W), V, k, _ptr(idx), _ptr(val),
                                     _ptr(logits), _ptr(n_fixup), _ptr(ws), ws.numel() * ws.element_size()),
           "lm_head_topk")


# ------------------------------------------------------------------ grouping
def group_workspace_bytes(T: int, k: int, E: int) -> int:
    return _load().tmoe_group_workspace_bytes(T, k, E)


def group_by_expert(idx, E: int, counts, offsets, sorted_token, sorted_slot, pos, ws=None, stream=None) -> None:
    T, k = idx.shape
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_load().tmoe_group_by_expert(_stream(stream), _ptr(idx), T, k, E, _ptr(counts), _ptr(offsets),
                                    _ptr(sorted_token), _ptr(sorted_slot), _ptr(pos), _ptr(ws), nb),
           "group_by_expert")


# ----------------------------------------------------------- layer weights
class MoEWeights:
    """Device weights of one layer plus the C struct that describes them.

    gate_p / up_p: uint8 [E][stride_gu]; down_p: uint8 [E][stride_d] (tiled
    layout); gate_s, up_s: fp32 [E][I]; down_s: fp32 [E][H]; router_w fp32
    [E][H]; router_bias fp32 [E] or None. Keeps references to the tensors.
    """

    def __init__(self, router_w, router_bias, gate_p, up_p, down_p, gate_s, up_s, down_s, top_k: int = 8):
        self.tensors = (router_w, router_bias, gate_p, up_p, down_p, gate_s, up_s, down_s)
        E, H = router_w.shape
        I = gate_s.shape[1]
        self.hidden, self.inter, self.n_experts, self.top_k = H, I, E, top_k
        s = _abi.MoEWeightsStruct()
        s.hidden, s.inter, s.n_experts, s.top_k, s.reserved = H, I, E, top_k, 0
        s.router_w, s.router_bias = _ptr(router_w), _ptr(router_bias)
        s.gate_p, s.up_p, s.down_p = _ptr(gate_p), _ptr(up_p), _ptr(down_p)
        s.stride_gu = gate_p.shape[1] if gate_p.dim() == 2 else tiled_bytes(I, H)
        s.stride_d = down_p.shape[1] if down_p.dim() == 2 else tiled_bytes(H, I)
        s.gate_s, s.up_s, s.down_s = _ptr(gate_s), _ptr(up_s), _ptr(down_s)
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)


class AttnWeights:
    """Device weights of one attention half plus the C struct that describes them.

    qkv_p: uint8 tiled [(n_heads + 2 n_kv) head_dim][hidden]; qkv_s fp32 per
    row; o_p: uint8 tiled [hidden][n_heads head_dim]; o_s fp32 per row.
    window > 0: sliding layer with rotary on rotary_dim dimensions; 0: global
    layer without positional encoding. Keeps references to the tensors."""

    def __init__(self, qkv_p, qkv_s, o_p, o_s, window: int, hidden: int = 2048, n_heads: int = 16,
                 n_kv_heads: int = 4, head_dim: int = 128, rotary_dim: int = 64, rope_base: float = 10000.0):
        self.tensors = (qkv_p, qkv_s, o_p, o_s)
        self.hidden, self.n_heads, self.n_kv_heads, self.head_dim = hidden, n_heads, n_kv_heads, head_dim
        self.window, self.rotary_dim, self.rope_base = window, rotary_dim, rope_base
        s = _abi.AttnWeightsStruct()
        s.hidden, s.n_heads, s.n_kv_heads, s.head_dim = hidden, n_heads, n_kv_heads, head_dim
        s.rotary_dim, s.window, s.reserved, s.rope_base = rotary_dim, window, 0, rope_base
        s.qkv_p, s.qkv_s, s.o_p, s.o_s = _ptr(qkv_p), _ptr(qkv_s), _ptr(o_p), _ptr(o_s)
        self.struct = s

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def attention_workspace_bytes(T: int, W: AttnWeights) -> int:
    n = _load().tmoe_attention_workspace_bytes(T, W.ref)
    if n == 0:
        raise RuntimeError("attention_workspace_bytes: unsupported attention shape")
    return n


def kv_cache(W: AttnWeights, capacity: int):
    """Zeroed fp32 key and value caches, each [n_kv][capacity][head_dim]."""
    import torch

    k = torch.zeros((W.n_kv_heads, capacity, W.head_dim), dtype=torch.float32, device="cuda")
    v = torch.zeros((W.n_kv_heads, capacity, W.head_dim), dtype=torch.float32, device="cuda")
    return k, v


def attention_forward(W: AttnWeights, X, pos0: int, k_cache, v_cache, ws, O=None, X_out=None, stream=None) -> None:
    """The attention half for T = X.shape[0] new tokens at positions pos0.. (X bf16 bit patterns)."""
    T = X.shape[0]
    cap = k_cache.shape[1]
    _check(_load().tmoe_attention_forward(_stream(stream), W.ref, _ptr(X), T, pos0, _ptr(k_cache), _ptr(v_cache), cap,
                                          _ptr(O), _ptr(X_out), _ptr(ws), ws.numel() * ws.element_size()),
           "attention_forward")


class HostBuffer:
    """Page-locked host memory that kernels read in place over PCIe
    (tmoe_host_alloc): `host` is its CPU address, `device` the address kernels
    use. Freed when the object is collected."""

    def __init__(self, nbytes: int):
        lib = _load()
        h, d = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib.tmoe_host_alloc(nbytes, ctypes.byref(h), ctypes.byref(d)), "host_alloc")
        self._free = lib.tmoe_host_free
        self.nbytes, self.host, self.device = int(nbytes), h.value, d.value

    def view(self, offset: int, nbytes: int):
        """A CPU uint8 tensor over bytes [offset, offset + nbytes) of the buffer."""
        import torch

        if offset < 0 or nbytes < 0 or offset + nbytes > self.nbytes:
            raise ValueError("view outside the host buffer")
        arr = (ctypes.c_uint8 * nbytes).from_address(self.host + offset)
        return torch.frombuffer(arr, dtype=torch.uint8)

    def __del__(self):
        if getattr(self, "host", None):
            self._free(self.host)
            self.host = None


def experts_on_host(W: MoEWeights) -> MoEWeights:
    """The same layer with its experts (packed gate/up/down and their row
    scales) copied into one pinned host buffer that the kernels read over PCIe
    on demand; the router stays in device memory. Results are bit-identical to
    W's: the same kernels run, only the experts' address space differs."""
    import torch

    router_w, router_bias, gate_p, up_p, down_p, gate_s, up_s, down_s = W.tensors
    parts = (gate_p, up_p, down_p, gate_s, up_s, down_s)
    offs, total = [], 0
    for t in parts:
        offs.append(total)
        total += (t.numel() * t.element_size() + 255) // 256 * 256
    buf = HostBuffer(total)
    for t, o in zip(parts, offs):
        buf.view(o, t.numel() * t.element_size()).copy_(t.contiguous().view(-1).view(torch.uint8))
    out = MoEWeights.__new__(MoEWeights)
    out.tensors = (router_w, router_bias)
    out.host_buffer = buf
    out.hidden, out.inter, out.n_experts, out.top_k = W.hidden, W.inter, W.n_experts, W.top_k
    s = _abi.MoEWeightsStruct()
    ctypes.memmove(ctypes.byref(s), ctypes.byref(W.struct), ctypes.sizeof(s))
    s.gate_p, s.up_p, s.down_p, s.gate_s, s.up_s, s.down_s = (buf.device + o for o in offs)
    out.struct = s
    return out


def ffn_workspace_bytes(T: int, W: MoEWeights) -> int:
    return _load().tmoe_ffn_workspace_bytes(T, W.ref)


def expert_ffn(W: MoEWeights, X, offsets, sorted_token, O, ws, clamp: float = 7.0, Hout=None, stream=None) -> None:
    T = X.shape[0]
    _check(_load().tmoe_expert_ffn(_stream(stream), W.ref, _ptr(X), T, _ptr(offsets), _ptr(sorted_token), clamp, _ptr(O),
                               _ptr(Hout), _ptr(ws), ws.numel() * ws.element_size()), "expert_ffn")


def combine(O, w, pos, Y=None, resid_in=None, resid_out=None, stream=None) -> None:
    T, k = w.shape
    H = O.shape[1]
    _check(_load().tmoe_combine(_stream(stream), _ptr(O), _ptr(w), _ptr(pos), T, k, H, _ptr(Y), _ptr(resid_in),
                            _ptr(resid_out)), "combine")


def moe_workspace_bytes(T: int, W: MoEWeights) -> int:
    out = ctypes.c_size_t(0)
    _check(_load().tmoe_moe_workspace_bytes(T, W.ref, ctypes.byref(out)), "moe_workspace_bytes")
    return out.value


def moe_forward(W: MoEWeights, X, Y, ws, clamp: float = 7.0, idx=None, w=None, pos=None, n_fixup=None,
                resid_out=None, stream=None) -> None:
    opt = _abi.MoEOptionsStruct()
    opt.clamp = clamp
    opt.reserved0 = 0
    opt.idx, opt.w, opt.pos, opt.n_fixup, opt.resid_out = _ptr(idx), _ptr(w), _ptr(pos), _ptr(n_fixup), _ptr(resid_out)
    T = X.shape[0]
    _check(_load().tmoe_moe_forward(_stream(stream), W.ref, _ptr(X), T, _ptr(Y), ctypes.byref(opt), _ptr(ws),
                                ws.numel() * ws.element_size()), "moe_forward")


NOALLOC_SCRATCH_BYTES = 32 << 20  # TMOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(W: MoEWeights, X, Y, clamp: float = 7.0, idx=None, w=None, pos=None, n_fixup=None,
                        resid_out=None, stream=None) -> None:
    """moe_forward without a caller workspace: the library's fixed per-GPU
    scratch array serves as the workspace (calls on one GPU must not overlap)."""
    opt = _abi.MoEOptionsStruct()
    opt.clamp = clamp
    opt.reserved0 = 0
    opt.idx, opt.w, opt.pos, opt.n_fixup, opt.resid_out = _ptr(idx), _ptr(w), _ptr(pos), _ptr(n_fixup), _ptr(resid_out)
    T = X.shape[0]
    _check(_load().tmoe_moe_forward_noalloc(_stream(stream), W.ref, _ptr(X), T, _ptr(Y), ctypes.byref(opt)),
           "moe_forward_noalloc")


# ------------------------------------------------------------- kernel timing
def profile_begin(kernel: str, capacity: int) -> None:
    """Start recording HIP events around each launch of `kernel` (see _abi.KERNELS)."""
    _check(_load().tmoe_profile_begin(_abi.KERNELS[kernel], capacity), "profile_begin")


def profile_end(capacity: int) -> np.ndarray:
    """Wait for the recorded launches and return their durations in milliseconds."""
    ms = np.zeros(max(capacity, 1), np.float32)
    n = ctypes.c_int(0)
    _check(_load().tmoe_profile_end(ms.ctypes.data_as(ctypes.c_void_p), capacity, ctypes.byref(n)), "profile_end")
    return ms[: n.value].copy()
