"""Synthetic layer weights built in HBM with the library's own device steps.

Raw fp32 weights come from the counter-based generator (tmoe_synth_ih12,
Philox4x64-10 + Irwin-Hall(12), the stream numbering of tmoe_inputs); each
expert matrix is then ternarized and packed on the device (tmoe_ternarize_pack)
and converted to the tiled layout (tmoe_repack_tiled). No host round trip.
"""
from __future__ import annotations

import numpy as np
import torch

import tmoe_inputs as ti

from . import MoEWeights, repack_tiled, synth_ih12, ternarize_pack, tiled_bytes


def _mat(cfg: int, layer: int, e: int, mat: int, rows: int, cols: int, wbuf, pbuf, out_tiled, out_s) -> None:
    w = wbuf[: rows * cols]
    synth_ih12(w, ti.stream_id(cfg, layer, e, mat))
    p = pbuf[: rows * ((cols + 4) // 5)].view(rows, (cols + 4) // 5)
    ternarize_pack(w.view(rows, cols), p, out_s)
    repack_tiled(p, cols, out_tiled)


def build_layer(cfg: int, layer: int, bias_kind: str | None = None, experts: int = ti.N_EXPERTS,
                hidden: int = ti.HIDDEN, inter: int = ti.INTER, top_k: int = ti.TOP_K) -> MoEWeights:
    dev = torch.device("cuda")
    E, H, I = experts, hidden, inter
    sgu, sd = tiled_bytes(I, H), tiled_bytes(H, I)
    gate_p = torch.empty((E, sgu), dtype=torch.uint8, device=dev)
    up_p = torch.empty((E, sgu), dtype=torch.uint8, device=dev)
    down_p = torch.empty((E, sd), dtype=torch.uint8, device=dev)
    gate_s = torch.empty((E, I), dtype=torch.float32, device=dev)
    up_s = torch.empty((E, I), dtype=torch.float32, device=dev)
    down_s = torch.empty((E, H), dtype=torch.float32, device=dev)
    wbuf = torch.empty(H * I, dtype=torch.float32, device=dev)
    pbuf = torch.empty(max(I * ((H + 4) // 5), H * ((I + 4) // 5)), dtype=torch.uint8, device=dev)
    for e in range(E):
        _mat(cfg, layer, e, ti.MAT_GATE, I, H, wbuf, pbuf, gate_p[e], gate_s[e])
        _mat(cfg, layer, e, ti.MAT_UP, I, H, wbuf, pbuf, up_p[e], up_s[e])
        _mat(cfg, layer, e, ti.MAT_DOWN, H, I, wbuf, pbuf, down_p[e], down_s[e])
    router_w = torch.empty((E, H), dtype=torch.float32, device=dev)
    synth_ih12(router_w.view(-1), ti.stream_id(cfg, layer, 1023, ti.MAT_ROUTER), mult=float(ti.ROUTER_STD))
    b = ti.router_bias(cfg, bias_kind, E)
    router_bias = None if b is None else torch.from_numpy(b).to(dev)
    return MoEWeights(router_w, router_bias, gate_p, up_p, down_p, gate_s, up_s, down_s, top_k=top_k)


def streamed_linear(cfg: int = 1, mats: int = 2048, rows: int = ti.INTER, cols: int = ti.HIDDEN):
    """`mats` distinct [rows][cols] ternary matrices stacked into one tiled
    [mats * rows][cols] matrix (tiled bytes and fp32 row scales on the device);
    matrix q takes the Philox stream (cfg, layer q // 1024, expert q % 1024,
    gate), so matrix 0 is the config's single linear matrix; each is
    ternarized and packed like every expert matrix."""
    dev = torch.device("cuda")
    Pt = torch.empty((mats, tiled_bytes(rows, cols)), dtype=torch.uint8, device=dev)
    s = torch.empty((mats, rows), dtype=torch.float32, device=dev)
    wbuf = torch.empty(rows * cols, dtype=torch.float32, device=dev)
    pbuf = torch.empty(rows * ((cols + 4) // 5), dtype=torch.uint8, device=dev)
    for q in range(mats):
        _mat(cfg, q // 1024, q % 1024, ti.MAT_GATE, rows, cols, wbuf, pbuf, Pt[q], s[q])
    return Pt.view(-1), s.view(-1)


def is_global_layer(layer: int) -> bool:
    """Layer pattern: three sliding-window layers, then one global layer
    (global at 3, 7, 11, 15, 19, 23: ai.thesatyajit.com, "The architecture
    around the quantization")."""
    return layer % 4 == 3


def build_attention(cfg: int, layer: int, global_layer: bool, window: int = 512, hidden: int = ti.HIDDEN):
    """The attention half of one layer: [q; k; v] (16 + 2 x 4 heads of 128) and
    output projections drawn as fp32(0.02) * IH12 (the streams of
    tmoe_inputs.attn_qkv_matrix / attn_o_matrix), ternarized and packed on the
    device. Global layers have no window and no rotary embedding."""
    from . import AttnWeights

    dev = torch.device("cuda")
    rows = ti.ATTN_QKV_ROWS
    qkv_p = torch.empty(tiled_bytes(rows, hidden), dtype=torch.uint8, device=dev)
    o_p = torch.empty(tiled_bytes(hidden, hidden), dtype=torch.uint8, device=dev)
    qkv_s = torch.empty(rows, dtype=torch.float32, device=dev)
    o_s = torch.empty(hidden, dtype=torch.float32, device=dev)
    w = torch.empty(rows * hidden, dtype=torch.float32, device=dev)
    p = torch.empty(rows * ((hidden + 4) // 5), dtype=torch.uint8, device=dev)
    for sid, R, out_p, out_s in ((ti.stream_id(cfg, layer, 0, ti.MAT_ATTN_QKV), rows, qkv_p, qkv_s),
                                 (ti.stream_id(cfg, layer, 0, ti.MAT_ATTN_O), hidden, o_p, o_s)):
        synth_ih12(w[: R * hidden], sid, mult=float(ti.ATTN_STD))
        pv = p[: R * ((hidden + 4) // 5)].view(R, (hidden + 4) // 5)
        ternarize_pack(w[: R * hidden].view(R, hidden), pv, out_s)
        repack_tiled(pv, hidden, out_p)
    return AttnWeights(qkv_p, qkv_s, o_p, o_s, window=0 if global_layer else window)


def activations(cfg: int, tokens: int, hidden: int = ti.HIDDEN, layer: int = 0) -> torch.Tensor:
    """bf16 activations as an int16 device tensor of bit patterns [T][H]."""
    x = ti.activations(cfg, tokens, hidden, layer)
    return torch.from_numpy(x.view(np.int16)).to("cuda")


def lm_head_table(cfg: int, vocab: int = ti.VOCAB, hidden: int = ti.HIDDEN) -> torch.Tensor:
    """The bf16 output embedding [vocab][hidden] on the device, as int16 bit
    patterns, bit-identical to tmoe_inputs.lm_head_rows (same Philox stream,
    fp32 scale, nearest-even rounding to bf16)."""
    w = torch.empty(vocab * hidden, dtype=torch.float32, device="cuda")
    synth_ih12(w, ti.stream_id(cfg, 0, 0, ti.MAT_LMHEAD), mult=float(ti.LMHEAD_STD))
    out = w.to(torch.bfloat16).view(torch.int16).view(vocab, hidden)
    del w
    return out

