"""Feeds seeded layer inputs (torch tensors in their storage formats) to the
oracle. TEST INFRASTRUCTURE ONLY, like the rest of oracle/.

Tensors are handed over as raw bits and decoded by the oracle's own exact
decoders (bf16, e4m3 with 128x128 block scales); nothing here computes any
step of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe_oracle as O


def decode_tensor(t: torch.Tensor, scale: torch.Tensor | None = None) -> np.ndarray:
    """Exact float64 values of a stored tensor. Large bf16 and e4m3 tensors
    (expert weights) are widened by torch's conversions, which equal the
    oracle's own decoders on every code (pinned over all 65536 bf16 and all
    256 e4m3 codes) and run on every host core; small ones go through the
    oracle's decoders themselves."""
    t = t.detach().cpu()
    big = t.numel() >= (1 << 20)
    if t.dtype == torch.float32:
        return O.decode_f32(t.numpy())
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy() if big else O.decode_bf16(t.view(torch.int16).numpy())
    if t.dtype == torch.uint8:
        if scale is None:
            raise ValueError("e4m3 codes need their block scales")
        sc = scale.detach().cpu().numpy()
        if big:
            return O.apply_block_scales(t.contiguous().view(torch.float8_e4m3fn).to(torch.float64).numpy(), sc)
        return O.dequant_e4m3_blocks(t.numpy(), sc)
    raise TypeError(t.dtype)


def router_params(cfg) -> O.RouterParams:
    return O.RouterParams(E=cfg.E, K=cfg.K, G=cfg.G, kg=cfg.kg, score_fn=cfg.score_fn,
                          norm=cfg.norm, rsf=cfg.rsf)


def routed_expert_fn(w):
    def get(e: int):
        gu = decode_tensor(w.gate_up[e], None if w.gate_up_scale is None else w.gate_up_scale[e])
        dn = decode_tensor(w.down[e], None if w.down_scale is None else w.down_scale[e])
        wg, wu = O.split_gate_up(gu)
        return wg, wu, dn
    return get


def shared_expert_fn(w):
    def get():
        if w is None:
            return None
        gu = decode_tensor(w.gate_up, w.gate_up_scale)
        dn = decode_tensor(w.down, w.down_scale)
        wg, wu = O.split_gate_up(gu)
        return wg, wu, dn
    return get


def route_inputs(inp) -> dict:
    u = decode_tensor(inp.x)
    bias = None if inp.sel_bias is None else decode_tensor(inp.sel_bias)
    return O.route(u, decode_tensor(inp.gate_w), bias, router_params(inp.cfg))


def run_layer(inp, tokens=None, routing=None, with_shared=True, add_residual=None):
    """Oracle output for `tokens` (default all) of a moe_inputs.LayerInputs."""
    u = decode_tensor(inp.x)
    bias = None if inp.sel_bias is None else decode_tensor(inp.sel_bias)
    r = inp.cfg.add_residual if add_residual is None else add_residual
    shared = shared_expert_fn(inp.shared) if (with_shared and inp.shared is not None) else None
    return O.layer_forward(router_params(inp.cfg), u, decode_tensor(inp.gate_w), bias,
                           routed_expert_fn(inp.experts), shared, add_residual=r,
                           tokens=tokens, routing=routing, act_quant=inp.cfg.act_quant)
