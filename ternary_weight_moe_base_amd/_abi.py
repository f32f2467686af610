"""ctypes declarations mirroring include/tmoe.h."""
import ctypes
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint64, c_void_p

TMOE_OK = 0
TMOE_E_ARG = -1
TMOE_E_SHAPE = -2
TMOE_E_ALIGN = -3
TMOE_E_BADPACK = -4
TMOE_E_WORKSPACE = -5
TMOE_E_UNSUPPORTED = -6
TMOE_E_HIP = -7

_NAMES = {0: "TMOE_OK", -1: "TMOE_E_ARG", -2: "TMOE_E_SHAPE", -3: "TMOE_E_ALIGN", -4: "TMOE_E_BADPACK",
          -5: "TMOE_E_WORKSPACE", -6: "TMOE_E_UNSUPPORTED", -7: "TMOE_E_HIP"}

_lib = None


def status_name(code: int) -> str:
    if _lib is not None:
        return _lib.tmoe_status_str(code).decode()
    return _NAMES.get(code, "TMOE_E_UNKNOWN")


def bind_status(lib) -> None:
    global _lib
    _lib = lib


class MoEWeightsStruct(ctypes.Structure):
    _fields_ = [
        ("hidden", c_int64), ("inter", c_int64), ("n_experts", c_int64), ("top_k", c_int32), ("reserved", c_int32),
        ("router_w", c_void_p), ("router_bias", c_void_p),
        ("gate_p", c_void_p), ("up_p", c_void_p), ("down_p", c_void_p),
        ("stride_gu", c_int64), ("stride_d", c_int64),
        ("gate_s", c_void_p), ("up_s", c_void_p), ("down_s", c_void_p),
    ]


class AttnWeightsStruct(ctypes.Structure):
    _fields_ = [
        ("hidden", c_int64), ("n_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
        ("rotary_dim", c_int32), ("window", c_int32), ("reserved", c_int32), ("rope_base", ctypes.c_double),
        ("qkv_p", c_void_p), ("qkv_s", c_void_p), ("o_p", c_void_p), ("o_s", c_void_p),
    ]


class MoEOptionsStruct(ctypes.Structure):
    _fields_ = [
        ("clamp", c_float), ("reserved0", c_int32),
        ("idx", c_void_p), ("w", c_void_p), ("pos", c_void_p), ("n_fixup", c_void_p), ("resid_out", c_void_p),
    ]


# name -> (restype, argtypes); every symbol declared in include/tmoe.h
SIGNATURES = {
    "tmoe_status_str": (c_char_p, [c_int]),
    "tmoe_last_error": (c_char_p, []),
    "tmoe_version": (c_int, []),
    "tmoe_ternarize_absmean_host": (c_int, [c_void_p, c_int64, c_int64, c_void_p, c_void_p]),
    "tmoe_pack_host": (c_int, [c_void_p, c_int64, c_int64, c_void_p, c_int64]),
    "tmoe_unpack_host": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "tmoe_validate_packed_host": (c_int, [c_void_p, c_int64, c_int64, c_int64, POINTER(c_int64)]),
    "tmoe_tiled_bytes": (c_int64, [c_int64, c_int64]),
    "tmoe_ternarize_pack": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_void_p]),
    "tmoe_unpack": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "tmoe_repack_tiled": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "tmoe_unpack_tiled": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p]),
    "tmoe_synth_ih12": (c_int, [c_void_p, c_uint64, c_uint64, c_uint64, c_uint64, c_int64, c_float, c_void_p]),
    "tmoe_linear_workspace_bytes": (c_size_t, [c_int64, c_int64]),
    "tmoe_ternary_linear": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64,
                                    c_void_p, c_int64, c_void_p, c_size_t]),
    "tmoe_linear_packed_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int64]),
    "tmoe_ternary_linear_packed": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_int64,
                                           c_int64, c_void_p, c_int64, c_void_p, c_size_t]),
    "tmoe_router_workspace_bytes": (c_size_t, [c_int64, c_int64]),
    "tmoe_router_topk": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_int, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t]),
    "tmoe_group_workspace_bytes": (c_size_t, [c_int64, c_int, c_int64]),
    "tmoe_group_by_expert": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_int64, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t]),
    "tmoe_ffn_workspace_bytes": (c_size_t, [c_int64, c_void_p]),
    "tmoe_expert_ffn": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_float, c_void_p,
                                c_void_p, c_void_p, c_size_t]),
    "tmoe_combine": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int64, c_void_p, c_void_p,
                             c_void_p]),
    "tmoe_moe_workspace_bytes": (c_int, [c_int64, c_void_p, POINTER(c_size_t)]),
    "tmoe_moe_forward": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_size_t]),
    "tmoe_moe_forward_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
    "tmoe_attention_workspace_bytes": (c_size_t, [c_int64, c_void_p]),
    "tmoe_attention_forward": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64,
                                       c_void_p, c_void_p, c_void_p, c_size_t]),
    "tmoe_host_alloc": (c_int, [c_size_t, POINTER(c_void_p), POINTER(c_void_p)]),
    "tmoe_host_free": (c_int, [c_void_p]),
    "tmoe_lm_head_workspace_bytes": (c_size_t, [c_int64, c_int64, c_int]),
    "tmoe_lm_head_topk": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_size_t]),
    "tmoe_profile_begin": (c_int, [c_int, c_int]),
    "tmoe_profile_end": (c_int, [c_void_p, c_int, POINTER(c_int)]),
}

KERNELS = {"router_logits": 1, "router_topk": 2, "group": 4, "make_tiles": 5, "gateup": 7, "down": 9, "combine": 10,
           "linear": 11, "lmh_logits": 12, "lmh_topk": 13, "lmh_merge": 14, "attention": 15}


def declare(lib) -> None:
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
