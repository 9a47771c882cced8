"""The layer under HIP graph capture (how a serving loop replays a decode
step): the cfg forward on the weight-streaming path (e4m3 weights, few
tokens) and on the grouped path (bf16, both router kernels), the
no-allocation forward, and a training step (the training forward and the
backward that reads what it kept). Each graph is replayed several times, with
the program's own eager calls and synchronisations between the replays, and
every replay is compared bit for bit with the eager result."""
import pytest
import torch

import mixture_experts_layer_38_amd as M
import moe_inputs as MI

pytestmark = pytest.mark.gpu

DEV = "cuda"

SMALL_FP8 = MI.LayerConfig("small_fp8", T=77, D=256, E=16, H=256, G=4, kg=2, K=4, score_fn="sigmoid",
                           bias="normal", norm=True, rsf=2.5, Hs=256, act="bf16", weight="fp8", bias_std=0.05)
# 400 tokens: the fp32 router kernel with split-K planes; 517: the bf16x3 router kernel
GROUPED_BF16 = MI.LayerConfig("grouped_bf16", T=400, D=384, E=32, H=256, G=8, kg=4, K=6, score_fn="sigmoid",
                              bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)
REPLAYS = 3


def _replays_match(step, outputs):
    """Eager reference of step() (after a warm-up on a side stream, as torch
    asks before a capture), then the captured step replayed REPLAYS times,
    each replay checked against it after the outputs are overwritten, with an
    eager call between the replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    step()
    torch.cuda.synchronize()
    ref = [o().clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outputs:
            t = o()
            t.fill_(float("nan") if t.is_floating_point() else -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(o(), r), (i, k)
        step()  # eager work between the replays
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("cfg,T", [(SMALL_FP8, 77), (GROUPED_BF16, 400), (GROUPED_BF16.with_(T=517), 517)],
                         ids=["stream_fp8", "grouped_bf16_fp32_router", "grouped_bf16_x3_router"])
def test_forward_replays_from_a_captured_graph(cfg, T):
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg)
    out = torch.empty((T, cfg.D), dtype=torch.float32, device=DEV)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=DEV)

    def step():
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out, expert_counts=counts)

    _replays_match(step, [lambda: out, lambda: counts])


def test_noalloc_forward_replays_from_a_captured_graph():
    cfg = SMALL_FP8
    inp = MI.make_layer(cfg, DEV)
    params = M.make_params(dim=cfg.D, n_routed=cfg.E, hidden=cfg.H, shared_hidden=cfg.Hs, top_k=cfg.K,
                           n_group=cfg.G, topk_group=cfg.kg, score_fn=cfg.score_fn, norm_topk=cfg.norm,
                           routed_scaling_factor=cfg.rsf, act=cfg.act, weight=cfg.weight, out=cfg.out,
                           add_residual=cfg.add_residual, max_tokens=0)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device=DEV)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=DEV)

    def step():
        M.layer_forward_noalloc(params, inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out,
                                expert_counts=counts)

    _replays_match(step, [lambda: out, lambda: counts])


def test_training_step_replays_from_a_captured_graph():
    cfg = GROUPED_BF16
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg, backward=True)
    d_out = torch.randn((cfg.T, cfg.D), generator=torch.Generator().manual_seed(4)).to(DEV)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device=DEV)
    grads = {}

    def step():
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out, train=True)
        g = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out, saved=True)
        if not grads:  # the first call's tensors are the ones every later call copies into
            grads.update({k: v for k, v in g.items() if v is not None})
        else:
            for k, v in grads.items():
                v.copy_(g[k])

    _replays_match(step, [lambda: out] + [(lambda k=k: grads[k]) for k in
                                         ("dx", "d_gate_w", "d_gate_up", "d_down", "d_shared_gate_up",
                                          "d_shared_down")])
