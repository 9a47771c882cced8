"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Sizes: small layers that span several tiles with ragged tails (both expert
GEMM paths), every workload at its full size (routing on all tokens; outputs
on all tokens where the oracle finishes in seconds, else on a seeded token
sample), and the edge cases (no tokens, one token, the maximum token count,
repeat-run bit identity, bf16 output, routed-only runs).
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_38_amd as M
import moe_inputs as MI
from oracle import adapter as A
from oracle import moe_oracle as O
from tests.parity import TOL, check_routing, layer_error, near_tie_mask

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_layer(inp, path="auto", with_shared=True, add_residual=None, out_dtype=None, T=None):
    cfg = inp.cfg
    over = {}
    if not with_shared:
        over["shared_hidden"] = 0
    if add_residual is not None:
        over["add_residual"] = add_residual
    if out_dtype is not None:
        over["out"] = out_dtype
    layer = M.MoELayer.from_config(cfg, path=path, **over)
    counts = torch.full((cfg.E,), -1, dtype=torch.int32, device=DEV)
    x = inp.x if T is None else inp.x[:T]
    out = layer.forward(x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared if with_shared else None,
                        expert_counts=counts)
    torch.cuda.synchronize()
    return out, counts, layer


def _sample(T, n, seed=7):
    if n >= T:
        return np.arange(T)
    return np.sort(np.random.default_rng(seed).choice(T, size=n, replace=False))


def _cover_experts(R, E, n_random=0, T=None, seed=7):
    """Tokens that put every expert with rows into the sample, at both ends
    of its rows: rows of an expert hold its tokens in ascending order, so its
    first and last token land in its first and its last (ragged) row tile;
    plus n_random seeded tokens."""
    idx = R["idx"]
    T = idx.shape[0] if T is None else T
    pick = set(_sample(T, n_random, seed).tolist()) if n_random else set()
    for e in range(E):
        tt = np.nonzero((idx == e).any(axis=1))[0]
        if tt.size:
            pick.update((int(tt[0]), int(tt[-1])))
    return np.array(sorted(pick), dtype=np.int64)


def _shared_ref(inp, tokens):
    """The shared expert's output for `tokens` (oracle FFN on the decoded
    weights; the e4m3-activation form when the layer quantises activations)."""
    sw = A.shared_expert_fn(inp.shared)()
    u = A.decode_tensor(inp.x)[tokens]
    ffn = O.swiglu_ffn_e4m3_act if inp.cfg.act_quant else O.swiglu_ffn
    return ffn(u, *sw)


def _check_layer(inp, tokens=None, path="auto", routed_only=True, compose=False, R=None):
    """Routing on every token, outputs on `tokens` (default all): the full
    layer and, if routed_only, a routed-only run (no shared expert, no
    residual) against the oracle. compose=True evaluates the oracle's routed
    part once and forms the full layer's reference as u + shared FFN + routed
    part (the output definition), so each expert's weights are decoded once."""
    cfg = inp.cfg
    R = A.route_inputs(inp) if R is None else R
    tokens = np.arange(cfg.T) if tokens is None else tokens
    near = near_tie_mask(R)[tokens]
    x64 = A.decode_tensor(inp.x)[tokens]
    out, counts, layer = _run_layer(inp, path=path)
    idx, gate, rc = layer.router(inp.x, inp.gate_w, inp.sel_bias)
    torch.cuda.synchronize()
    info = check_routing(idx, gate, rc, R, cfg.E, cfg.G, cfg.kg)
    assert torch.equal(counts, rc)
    tsel = torch.as_tensor(tokens, device=DEV)
    tol = TOL[cfg.weight]
    ref_r = None
    if compose:
        ref_r, _ = A.run_layer(inp, tokens=tokens, routing=R, with_shared=False, add_residual=False)
        ref = ref_r + (x64 if cfg.add_residual else 0.0)
        if inp.shared is not None:
            ref = ref + _shared_ref(inp, tokens)
    else:
        ref, _ = A.run_layer(inp, tokens=tokens, routing=R)
    err = layer_error(out[tsel], ref, x64, cfg.add_residual, exclude=near)
    print(f"{cfg.name} path={path}: routing {info}, full layer err {err} on {len(tokens)} tokens")
    assert err["max"] <= tol, err
    if routed_only:
        del out
        out_r, _, _ = _run_layer(inp, path=path, with_shared=False, add_residual=False)
        if ref_r is None:
            ref_r, _ = A.run_layer(inp, tokens=tokens, routing=R, with_shared=False, add_residual=False)
        err_r = layer_error(out_r[tsel], ref_r, x64, False, exclude=near)
        print(f"{cfg.name} path={path}: routed-only err {err_r}")
        assert err_r["max"] <= tol, err_r
    return info, err


# ---------------------------------------------------------------------------
# small layers: several tiles, ragged tails
# ---------------------------------------------------------------------------

SMALL_BF16 = MI.LayerConfig("small_bf16", T=300, D=256, E=16, H=128, G=4, kg=2, K=3, score_fn="softmax",
                            bias="none", norm=False, rsf=1.0, Hs=256, act="bf16", weight="bf16")
SMALL_SIG = MI.LayerConfig("small_sigmoid", T=517, D=384, E=32, H=256, G=8, kg=4, K=6, score_fn="sigmoid",
                           bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)
SMALL_FP8 = MI.LayerConfig("small_fp8", T=77, D=256, E=16, H=256, G=4, kg=2, K=4, score_fn="sigmoid",
                           bias="normal", norm=True, rsf=2.5, Hs=256, act="bf16", weight="fp8", bias_std=0.05)
SMALL_F32 = MI.LayerConfig("small_f32", T=129, D=96, E=10, H=48, G=2, kg=1, K=3, score_fn="softmax",
                           bias="none", norm=False, rsf=1.5, Hs=40, act="f32", weight="f32")
# bf16 activations from 512 tokens on take the bf16x3 logits kernel: 9 ragged token
# tiles, a second expert tile holding 8 of its 128 experts, several K splits
ROUTER_X3 = MI.LayerConfig("router_x3", T=1100, D=512, E=136, H=128, G=8, kg=3, K=5, score_fn="sigmoid",
                           bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)
ROUTER_X3_SOFTMAX = MI.LayerConfig("router_x3_softmax", T=640, D=256, E=64, H=128, G=1, kg=1, K=6,
                                   score_fn="softmax", bias="none", norm=False, rsf=1.0, Hs=128, act="bf16",
                                   weight="bf16")
# more than 256 experts: eight values per lane in the select kernel, three expert tiles
ROUTER_E384 = MI.LayerConfig("router_e384", T=700, D=256, E=384, H=128, G=12, kg=4, K=8, score_fn="sigmoid",
                             bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)


def test_generator_is_device_agnostic():
    k = MI.stream_key(0, MI.TID_GATE_UP)
    a = MI.uniform_pm(k, 12345, (300, 128), 0.03, "cpu")
    b = MI.uniform_pm(k, 12345, (300, 128), 0.03, DEV).cpu()
    assert torch.equal(a, b)


def test_router_small_all_score_functions():
    # ROUTER_E384 at 100 tokens: split-K planes added by the selection kernel
    # with one token per workgroup and eight values per lane
    for cfg in (SMALL_BF16, SMALL_SIG, SMALL_F32, MI.CONFIGS["tiny_f32"], ROUTER_X3, ROUTER_X3_SOFTMAX,
                ROUTER_E384, ROUTER_E384.with_(name="router_e384_few", T=100)):
        inp = MI.make_layer(cfg, DEV)
        layer = M.MoELayer.from_config(cfg)
        idx, gate, counts = layer.router(inp.x, inp.gate_w, inp.sel_bias)
        torch.cuda.synchronize()
        info = check_routing(idx, gate, counts, A.route_inputs(inp), cfg.E, cfg.G, cfg.kg)
        # canonical order: descending selection score
        R = A.route_inputs(inp)
        zsel = np.take_along_axis(R["z"], idx.cpu().numpy().astype(np.int64), 1)
        assert np.all(np.diff(zsel, axis=1) <= 2e-6)
        print(cfg.name, info)


def test_router_forced_expert_and_all_ties():
    cfg = SMALL_SIG
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg)
    b = torch.zeros(cfg.E, device=DEV)
    b[13] = 10.0
    idx, gate, counts = layer.router(inp.x, inp.gate_w, b)
    torch.cuda.synchronize()
    assert int(counts[13]) == cfg.T
    assert bool((idx == 13).any(dim=1).all())
    # x = 0: every score equal -> lowest groups, lowest indices
    x0 = torch.zeros_like(inp.x)
    idx, gate, counts = layer.router(x0, inp.gate_w, None)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), torch.arange(cfg.K, dtype=torch.int32).expand(cfg.T, cfg.K))
    assert torch.allclose(gate.cpu(), torch.full((cfg.T, cfg.K), cfg.rsf / cfg.K))


def test_dispatch_is_the_stable_permutation():
    """Rows by the definition: (t, k) with expert e goes to offsets[e] plus the
    number of earlier entries with expert e (batches of up to 1024 entries take
    the one-workgroup path, larger ones the chunked one: both sides of that
    boundary, a skewed case where one expert takes most tokens, and E = 512)."""
    rng = np.random.default_rng(3)
    for cfg, Ts in ((SMALL_SIG, (1, 77, 170, 171, 517, 1400)), (ROUTER_E384.with_(E=512, G=16, kg=4), (128, 129, 900))):
        layer = M.MoELayer.from_config(cfg.with_(T=max(Ts)))
        for T in Ts:
            for skew in (False, True):
                p = np.ones(cfg.E)
                if skew:
                    p[3] = 50.0 * cfg.E
                p /= p.sum()
                idx = np.stack([rng.choice(cfg.E, size=cfg.K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
                off, row_token, slot_row = layer.dispatch(torch.from_numpy(idx).to(DEV))
                torch.cuda.synchronize()
                off, row_token, slot_row = off.cpu().numpy(), row_token.cpu().numpy(), slot_row.cpu().numpy()
                cnt = np.bincount(idx.ravel(), minlength=cfg.E)
                assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
                seen = np.zeros(cfg.E, np.int64)
                want_slot = np.empty(T * cfg.K, np.int64)
                for i, e in enumerate(idx.ravel()):
                    want_slot[i] = off[e] + seen[e]
                    seen[e] += 1
                assert np.array_equal(slot_row, want_slot)
                assert np.array_equal(row_token[want_slot], np.arange(T * cfg.K) // cfg.K)


@pytest.mark.parametrize("cfg,path", [(SMALL_F32, "auto"), (MI.CONFIGS["tiny_f32"], "auto"),
                                      (SMALL_BF16, "grouped"), (SMALL_BF16, "stream"),
                                      (SMALL_SIG, "grouped"), (SMALL_SIG, "stream"), (SMALL_FP8, "stream"),
                                      (SMALL_FP8, "grouped")],
                         ids=lambda v: v if isinstance(v, str) else v.name)
def test_layer_small(cfg, path):
    inp = MI.make_layer(cfg, DEV)
    _check_layer(inp, path=path)


@pytest.mark.parametrize("K,path", [(1, "grouped"), (12, "grouped"), (16, "grouped"), (16, "stream")])
def test_layer_top_k_extremes(K, path):
    """The smallest and largest accepted top-K (1 and 16; 12 in between):
    the selection beyond 8 slots, the dispatch at T*K around the
    one-workgroup limit, and the combine's second group of row loads."""
    T = 64 if path == "stream" else 300
    cfg = MI.LayerConfig(f"topk{K}", T=T, D=256, E=64, H=128, G=8, kg=4, K=K, score_fn="sigmoid",
                         bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)
    inp = MI.make_layer(cfg, DEV)
    _check_layer(inp, path=path)


@pytest.mark.parametrize("path", ["stream", "grouped"])
def test_layer_fp8_every_code(path):
    """Expert weights drawn uniformly over all 254 finite e4m3 codes (tiny,
    subnormal and large values alike), so any mis-decoded code shows up."""
    cfg = SMALL_FP8
    inp = MI.make_layer(cfg, DEV)
    g = torch.Generator().manual_seed(5)

    def every_code(t):
        r = torch.randint(0, 254, t.shape, generator=g, dtype=torch.int32)
        r = torch.where(r >= 0x7F, r + 1, r)  # skip 0x7F; 0xFF is never reached
        t.copy_(r.to(torch.uint8).to(t.device))
    for w in (inp.experts.gate_up, inp.experts.down, inp.shared.gate_up, inp.shared.down):
        every_code(w)
    _check_layer(inp, path=path)


def test_layer_edge_cases():
    cfg = SMALL_SIG
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg)
    # T = 0 zeroes the counts and writes nothing
    counts = torch.full((cfg.E,), 7, dtype=torch.int32, device=DEV)
    out = torch.full((1, cfg.D), 3.0, device=DEV)
    layer.forward(inp.x[:0], inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out[:0], expert_counts=counts)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and bool((out == 3.0).all())
    # T = 1 and T = max_tokens agree with the oracle on those tokens
    R = A.route_inputs(inp)
    for T in (1, cfg.T):
        o = layer.forward(inp.x[:T].contiguous(), inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
        torch.cuda.synchronize()
        ref, _ = A.run_layer(inp, tokens=np.arange(T), routing=R)
        err = layer_error(o, ref, A.decode_tensor(inp.x)[:T], True, exclude=near_tie_mask(R)[:T])
        assert err["max"] <= TOL["bf16"]
    # T > max_tokens is rejected
    with pytest.raises(M.MoEError):
        big = torch.zeros((cfg.T + 1, cfg.D), dtype=torch.bfloat16, device=DEV)
        layer.forward(big, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    # repeat runs are bit-identical (no float atomics anywhere)
    o1 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    o2 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    # bf16 output is the fp32 output rounded
    ob, _, _ = _run_layer(inp, out_dtype="bf16")
    assert torch.equal(ob, o1.to(torch.bfloat16))


# e4m3 weights at a prefill token count: the grouped GEMMs widen them to bf16
# (times the block scale) as they stage them
FP8_PREFILL = MI.LayerConfig("fp8_prefill", T=2100, D=1024, E=32, H=512, G=4, kg=2, K=4, score_fn="sigmoid",
                             bias="normal", norm=True, rsf=2.5, Hs=512, act="bf16", weight="fp8", bias_std=0.02)


def test_layer_fp8_prefill():
    inp = MI.make_layer(FP8_PREFILL, DEV)
    _check_layer(inp, tokens=_sample(FP8_PREFILL.T, 200))


# e4m3 activations with 1x128 block scales on the fp8 matrix cores: token rows
# and h quantised, weights e4m3 with 128x128 block scales; 128-row tiles.
# small_w8a8: 2 K steps in both GEMMs; w8a8_odd: 3 K steps (a tail step) in
# the gate/up GEMM and the shared down GEMM, 1 in the routed down GEMM;
# w8a8_prefill: about 260 rows per expert, three row tiles each
SMALL_W8A8 = SMALL_FP8.with_(name="small_w8a8", act_quant=True)
W8A8_ODD = MI.LayerConfig("w8a8_odd", T=300, D=384, E=16, H=128, G=4, kg=2, K=3, score_fn="sigmoid",
                          bias="normal", norm=True, rsf=2.5, Hs=384, act="bf16", weight="fp8", bias_std=0.05,
                          act_quant=True)
W8A8_PREFILL = FP8_PREFILL.with_(name="w8a8_prefill", act_quant=True)


@pytest.mark.parametrize("cfg", [SMALL_W8A8, W8A8_ODD, W8A8_PREFILL], ids=lambda c: c.name)
def test_layer_e4m3_activations(cfg):
    inp = MI.make_layer(cfg, DEV)
    _check_layer(inp, tokens=_sample(cfg.T, 200))


# Bounds that tell the e4m3-activation kernels from ones that skip a
# quantisation step: on W8A8_PREFILL's sampled tokens the oracle without the
# token-row quantisation differs from the quantised oracle by a median e_t of
# 4.9e-2, without the h quantisation by 2.3e-2 (max 3.4e-2), while the
# kernels' own error (bf16 y slots, fp32 sum order) is about 2e-3 median.
W8A8_MEDIAN_BOUND = 8e-3
W8A8_MAX_BOUND = 1.5e-2


def _ffn_quant_variant(quant_u, quant_h):
    """The FFN with only the chosen GEMM inputs quantised (oracle steps)."""
    def qdq(v):
        return O.dequant_act_1x128(*O.quantize_act_1x128(np.asarray(v).astype(np.float32)))

    def f(u, wg, wu, wd):
        u = qdq(u) if quant_u else u
        h = O.silu(u @ wg.T) * (u @ wu.T)
        return (qdq(h) if quant_h else h) @ wd.T
    return f


def test_layer_w8a8_matches_each_quantisation_step():
    """Routed-only w8a8 layer: the GPU output is within the tight bounds of
    the quantised oracle, and each oracle variant that drops one quantisation
    step (token rows, h, or both) lies outside them."""
    cfg = W8A8_PREFILL
    inp = MI.make_layer(cfg, DEV)
    tokens = _sample(cfg.T, 200)
    R = A.route_inputs(inp)
    near = near_tie_mask(R)[tokens]
    out, _, _ = _run_layer(inp, with_shared=False, add_residual=False)
    got = out[torch.as_tensor(tokens, device=DEV)]
    u = A.decode_tensor(inp.x)[tokens]
    idx, gate = R["idx"][tokens], R["gate"][tokens]
    ex = A.routed_expert_fn(inp.experts)
    refs = {}
    for name, qu, qh in (("w8a8", 1, 1), ("tokens not quantised", 0, 1), ("h not quantised", 1, 0),
                         ("nothing quantised", 0, 0)):
        f = _ffn_quant_variant(qu, qh)
        Y = np.zeros((len(tokens), cfg.K, cfg.D))
        for e in np.unique(idx):
            ii, kk = np.nonzero(idx == e)
            Y[ii, kk] = f(u[ii], *ex(int(e)))
        refs[name] = sum(gate[:, k:k + 1] * Y[:, k] for k in range(cfg.K))
    # the variant built from the oracle's steps is the oracle's own layer output
    ref_layer, _ = A.run_layer(inp, tokens=tokens, routing=R, with_shared=False, add_residual=False)
    assert np.allclose(refs["w8a8"], ref_layer, rtol=1e-12, atol=1e-12)
    errs = {name: layer_error(got, ref, u, False, exclude=near) for name, ref in refs.items()}
    print(f"w8a8 GPU error against each oracle variant: {errs}")
    assert errs["w8a8"]["median"] <= W8A8_MEDIAN_BOUND and errs["w8a8"]["max"] <= W8A8_MAX_BOUND, errs["w8a8"]
    for name in ("tokens not quantised", "h not quantised", "nothing quantised"):
        assert errs[name]["median"] > W8A8_MEDIAN_BOUND, (name, errs[name])
        sep = layer_error(torch.from_numpy(refs[name]), refs["w8a8"], u, False, exclude=near)
        assert sep["median"] > 2 * W8A8_MEDIAN_BOUND, (name, sep)


def test_layer_e4m3_activations_every_code_and_edges():
    """Weights over all finite e4m3 codes; then T = 1 and T = max_tokens, and
    repeat runs bit-identical."""
    cfg = SMALL_W8A8
    inp = MI.make_layer(cfg, DEV)
    g = torch.Generator().manual_seed(9)
    for w in (inp.experts.gate_up, inp.experts.down, inp.shared.gate_up, inp.shared.down):
        r = torch.randint(0, 254, w.shape, generator=g, dtype=torch.int32)
        w.copy_(torch.where(r >= 0x7F, r + 1, r).to(torch.uint8).to(DEV))
    _check_layer(inp)
    layer = M.MoELayer.from_config(cfg)
    R = A.route_inputs(inp)
    for T in (1, cfg.T):
        o = layer.forward(inp.x[:T].contiguous(), inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
        torch.cuda.synchronize()
        ref, _ = A.run_layer(inp, tokens=np.arange(T), routing=R)
        err = layer_error(o, ref, A.decode_tensor(inp.x)[:T], True, exclude=near_tie_mask(R)[:T])
        assert err["max"] <= TOL["fp8"], (T, err)
    o1 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    o2 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def _quant_parity(x_bf16_cpu, rows=None):
    """GPU quantiser vs the oracle, bit for bit, on all rows or the given ones."""
    codes, scales = M.quantize_e4m3_1x128(x_bf16_cpu.to(DEV).contiguous())
    torch.cuda.synchronize()
    xs = x_bf16_cpu if rows is None else x_bf16_cpu[torch.as_tensor(rows)]
    rc, rs = O.quantize_act_1x128(O.decode_bf16(xs.view(torch.int16).numpy()).astype(np.float32))
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}"


def test_quantizer_matches_the_oracle_bit_for_bit():
    g = torch.Generator().manual_seed(11)
    rows, cols = 301, 1024
    mag = torch.logspace(-25, 25, rows, dtype=torch.float64)[:, None]
    x = (torch.randn((rows, cols), generator=g, dtype=torch.float64) * mag).to(torch.bfloat16)
    x[3] = 0.0                                   # all-zero blocks
    x[4] = -0.0                                  # negative zeros
    x[5, :] = 0.0
    x[5, 200] = -3.0                             # a single value per block
    # scale exactly 1 (block maximum 448) and every midpoint between two e4m3
    # values (exact in bf16): ties to the even code, each sign
    t = O.decode_e4m3(np.arange(0x7F))
    mids = torch.from_numpy(np.concatenate([[448.0], (t[:-1] + t[1:]) / 2, [-448.0]]))
    x[6] = torch.cat([mids, -mids]).repeat(cols // 256).to(torch.bfloat16)
    x[7] = torch.full((cols,), 448.0, dtype=torch.bfloat16)  # every value the block maximum
    _quant_parity(x)
    # a single row and an empty input
    _quant_parity(x[:1].clone())
    c0, s0 = M.quantize_e4m3_1x128(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV))
    assert c0.shape == (0, 256) and s0.shape == (0, 2)


# ---------------------------------------------------------------------------
# backward pass: gradients against the oracle's chain rule
# ---------------------------------------------------------------------------

BWD_SIG = MI.LayerConfig("bwd_sigmoid", T=300, D=256, E=16, H=128, G=4, kg=2, K=3, score_fn="sigmoid",
                         bias="normal", norm=True, rsf=2.5, Hs=256, act="bf16", weight="bf16", bias_std=0.05)
BWD_SOFTMAX = MI.LayerConfig("bwd_softmax", T=200, D=384, E=40, H=256, G=1, kg=1, K=4, score_fn="softmax",
                             bias="none", norm=False, rsf=1.5, Hs=128, act="bf16", weight="bf16")
BWD_GROUP = MI.LayerConfig("bwd_group", T=1000, D=1024, E=64, H=512, G=8, kg=3, K=6, score_fn="softmax",
                           bias="none", norm=False, rsf=1.0, Hs=1024, act="bf16", weight="bf16")


def _rel(a, b):
    a = a.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(a) else a
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def _rel_rows(a, b, floor=0.25):
    """Per-row error of a matrix: max over rows of max|a - b| / max(max|b|
    within the row, floor x the matrix maximum).

    A weight-gradient row is a sum of products with the bf16-rounded upstream
    gradient, so its error has an absolute size (a few 2^-9 of the matrix's
    typical entry), not one relative to the row: a row far below the matrix
    maximum cannot be held to the relative bound (with a 1 % floor the sparse
    case measures 0.05 - 0.12). With the floor at 1/4, a row that is dropped
    or garbled still fails once its size passes tolerance x floor (0.5 % of
    the matrix maximum at the bf16 tolerance), four times finer than the
    whole-matrix max|a - b| / max|b|."""
    a = a.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(a) else a
    a, b = a.reshape(a.shape[0], -1), np.asarray(b).reshape(b.shape[0], -1)
    den = np.maximum(np.abs(b).max(axis=1), floor * max(np.abs(b).max(), 1e-30))
    return float((np.abs(a - b).max(axis=1) / den).max())


def _check_backward(cfg, add_residual=True, with_shared=True, seed=5, inp=None):
    inp = MI.make_layer(cfg, DEV) if inp is None else inp
    over = {} if with_shared else {"shared_hidden": 0}
    layer = M.MoELayer.from_config(cfg, backward=True, add_residual=add_residual, **over)
    g = torch.Generator().manual_seed(seed)
    d_out = torch.randn((cfg.T, cfg.D), generator=g).to(DEV)
    shared = inp.shared if with_shared else None
    got = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, shared, d_out)
    torch.cuda.synchronize()
    R = A.route_inputs(inp)
    assert not near_tie_mask(R).any(), "a near-tie token: pick another seed for this case"
    u = A.decode_tensor(inp.x)
    bias = None if inp.sel_bias is None else A.decode_tensor(inp.sel_bias)
    ref = O.layer_backward(A.router_params(cfg), u, A.decode_tensor(inp.gate_w), bias,
                           A.routed_expert_fn(inp.experts), d_out.cpu().numpy().astype(np.float64),
                           A.shared_expert_fn(shared) if with_shared else None, add_residual=add_residual,
                           routing=R)
    tol = TOL["bf16"]
    dx = got["dx"].cpu().numpy().astype(np.float64)
    e_dx = np.abs(dx - ref["dx"]).max(axis=1) / np.maximum(np.abs(ref["dx"]).max(axis=1), 1e-30)
    errs = {"dx": float(e_dx.max()), "d_gate_w": _rel_rows(got["d_gate_w"], ref["d_gate_w"])}
    worst_w = 0.0
    for e in range(cfg.E):
        if e not in ref["d_routed"]:
            assert not got["d_gate_up"][e].any() and not got["d_down"][e].any(), f"unused expert {e} not zero"
            continue
        dwg, dwu, dwd = ref["d_routed"][e]
        worst_w = max(worst_w, _rel_rows(got["d_gate_up"][e], np.concatenate([dwg, dwu], 0)),
                      _rel_rows(got["d_down"][e], dwd))
    errs["d_experts"] = worst_w
    if with_shared:
        dwg, dwu, dwd = ref["d_shared"]
        errs["d_shared"] = max(_rel_rows(got["d_shared_gate_up"], np.concatenate([dwg, dwu], 0)),
                               _rel_rows(got["d_shared_down"], dwd))
    # the same rows against a 1 % floor, for the record: small rows carry the
    # absolute rounding error of the upstream gradient
    fine = {"d_gate_w": _rel_rows(got["d_gate_w"], ref["d_gate_w"], floor=1e-2)}
    print(f"{cfg.name} backward errors {errs}; 1 % floor: {fine}")
    for k, v in errs.items():
        assert v <= tol, (k, v)
    return layer, inp, d_out, got


# few tokens over many experts: about half the experts get no rows (zero
# weight gradients), and with ~1000 weight-gradient tiles each workgroup of
# the persistent weight-gradient grid walks several tiles, empty ones among them
BWD_SPARSE = MI.LayerConfig("bwd_sparse", T=40, D=1024, E=64, H=512, G=8, kg=3, K=2, score_fn="softmax",
                            bias="none", norm=True, rsf=1.0, Hs=512, act="bf16", weight="bf16")


@pytest.mark.parametrize("cfg", [BWD_SIG, BWD_SOFTMAX, BWD_GROUP, BWD_SPARSE], ids=lambda c: c.name)
def test_backward_matches_the_oracle(cfg):
    _check_backward(cfg)


def test_backward_routed_only_and_repeatable():
    layer, inp, d_out, g1 = _check_backward(BWD_SIG, add_residual=False, with_shared=False)
    g2 = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, None, d_out)
    torch.cuda.synchronize()
    for k in ("dx", "d_gate_w", "d_gate_up", "d_down"):
        assert torch.equal(g1[k], g2[k]), k  # no float atomics: bit-identical repeats
    # T = 0 zeroes every gradient
    g0 = layer.backward(inp.x[:0], inp.gate_w, inp.sel_bias, inp.experts, None, d_out[:0])
    torch.cuda.synchronize()
    assert not g0["d_gate_w"].any() and not g0["d_gate_up"].any() and not g0["d_down"].any()
    # T = 1: one row per chosen expert, every other expert zero
    x1, d1 = inp.x[:1].contiguous(), d_out[:1].contiguous()
    gt = layer.backward(x1, inp.gate_w, inp.sel_bias, inp.experts, None, d1)
    torch.cuda.synchronize()
    cfg = BWD_SIG
    bias = None if inp.sel_bias is None else A.decode_tensor(inp.sel_bias)
    ref = O.layer_backward(A.router_params(cfg), A.decode_tensor(inp.x)[:1], A.decode_tensor(inp.gate_w), bias,
                           A.routed_expert_fn(inp.experts), d1.cpu().numpy().astype(np.float64), None,
                           add_residual=False)
    assert _rel(gt["dx"], ref["dx"]) <= TOL["bf16"] and _rel_rows(gt["d_gate_w"], ref["d_gate_w"]) <= TOL["bf16"]
    for e in range(cfg.E):
        if e in ref["d_routed"]:
            dwg, dwu, dwd = ref["d_routed"][e]
            assert _rel_rows(gt["d_gate_up"][e], np.concatenate([dwg, dwu], 0)) <= TOL["bf16"]
            assert _rel_rows(gt["d_down"][e], dwd) <= TOL["bf16"]
        else:
            assert not gt["d_gate_up"][e].any() and not gt["d_down"][e].any()


SKEWED = MI.LayerConfig("skewed", T=1100, D=256, E=16, H=128, G=4, kg=2, K=3, score_fn="sigmoid",
                        bias="normal", norm=True, rsf=2.5, Hs=128, act="bf16", weight="bf16", bias_std=0.05)


# Every row count a tile body distinguishes: one expert per token (K = 1),
# the expert of each token forced through x and gate_w (gate_w[e] is the
# e-th unit vector, x carries 4.0 in the column of its expert and 0 in the
# other expert columns), so expert e holds exactly ROW_SWEEP[e] rows: 1 row,
# both sides of every 16-, 32- and 64-row boundary up to two 256-row tiles,
# and an expert with no rows. Each product's kernels then run tiles and items
# with every count of valid row blocks and of row groups to load.
ROW_SWEEP = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 127, 128, 129, 191, 192, 193, 255, 256, 257, 300, 511, 512,
             513, 700, 0]
SWEEP_BF16 = MI.LayerConfig("row_sweep_bf16", T=sum(ROW_SWEEP), D=256, E=len(ROW_SWEEP), H=256, G=1, kg=1, K=1,
                            score_fn="softmax", bias="none", norm=False, rsf=1.0, Hs=256, act="bf16",
                            weight="bf16")


def _forced_routing(inp, counts, seed=11):
    cfg = inp.cfg
    expert = np.repeat(np.arange(len(counts)), counts)
    np.random.default_rng(seed).shuffle(expert)  # an expert's tokens spread over the batch
    e_t = torch.as_tensor(expert, device=DEV)
    x = inp.x.clone()
    x[:, :cfg.E] = 0
    x[torch.arange(cfg.T, device=DEV), e_t] = 4.0
    gw = torch.zeros((cfg.E, cfg.D), dtype=torch.float32, device=DEV)
    gw[torch.arange(cfg.E), torch.arange(cfg.E)] = 1.0
    return dataclasses.replace(inp, x=x, gate_w=gw)


@pytest.mark.parametrize("cfg,path", [(SWEEP_BF16, "grouped"), (SWEEP_BF16, "stream"),
                                      (SWEEP_BF16.with_(name="row_sweep_fp8", weight="fp8"), "grouped"),
                                      (SWEEP_BF16.with_(name="row_sweep_fp8", weight="fp8"), "stream"),
                                      (SWEEP_BF16.with_(name="row_sweep_w8a8", weight="fp8", act_quant=True), "auto"),
                                      (SWEEP_BF16.with_(name="row_sweep_f32", act="f32", weight="f32"), "auto")],
                         ids=["bf16-grouped", "bf16-stream", "fp8-grouped", "fp8-stream", "w8a8", "f32"])
def test_layer_every_tile_row_count(cfg, path):
    inp = _forced_routing(MI.make_layer(cfg, DEV), ROW_SWEEP)
    R = A.route_inputs(inp)
    assert np.array_equal(np.bincount(R["idx"].ravel(), minlength=cfg.E), ROW_SWEEP)
    _check_layer(inp, path=path, R=R)


def test_backward_every_tile_row_count():
    """The backward's grouped products on the same forced routing: every
    count of valid row blocks in the data-gradient tiles, expert row counts
    on both sides of the 64-row K steps of the weight gradients, and an
    expert without rows (zero weight gradient)."""
    inp = _forced_routing(MI.make_layer(SWEEP_BF16, DEV), ROW_SWEEP)
    _check_backward(SWEEP_BF16, inp=inp)


def _train_step_matches(cfg, inp, seed=6):
    """The forward of a training step against the grouped-path forward, and
    the backward that reads its saved gate/up products against the one that
    recomputes them: both bit for bit (the same tile bodies and epilogue
    expressions produce h, [a | u] and g * h)."""
    layer = M.MoELayer.from_config(cfg, backward=True, path="grouped")
    out0 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    out1 = layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, train=True)
    d_out = torch.randn((cfg.T, cfg.D), generator=torch.Generator().manual_seed(seed)).to(DEV)
    g_saved = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out, saved=True)
    g_rec = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    for k, v in g_rec.items():
        if v is None:
            assert g_saved[k] is None, k
        else:
            assert torch.equal(v, g_saved[k]), k
    del layer


@pytest.mark.parametrize("name", ["small_sigmoid", "skewed", "row_sweep", "no_shared"])
def test_training_forward_and_saved_backward(name):
    """Ragged and skewed expert row counts (the row sweep: every count of
    valid row blocks, an expert without rows), with a shared expert, and a
    layer without one."""
    if name == "row_sweep":
        inp = _forced_routing(MI.make_layer(SWEEP_BF16, DEV), ROW_SWEEP)
    else:
        cfg = {"small_sigmoid": SMALL_SIG, "skewed": SKEWED,
               "no_shared": SMALL_SIG.with_(name="small_sigmoid_no_shared", Hs=0)}[name]
        inp = MI.make_layer(cfg, DEV)
    _train_step_matches(inp.cfg, inp)


def test_saved_backward_needs_its_training_forward():
    """No training forward yet, a different token count, or a recomputing
    backward in between: the saved backward refuses and launches nothing."""
    cfg = SMALL_SIG
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg, backward=True)
    d_out = torch.randn((cfg.T, cfg.D), generator=torch.Generator().manual_seed(2)).to(DEV)
    args = (inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
    with pytest.raises(M.MoEError):
        layer.backward(*args, d_out, saved=True)
    layer.forward(*args, train=True)
    with pytest.raises(M.MoEError):
        layer.backward(inp.x[:100].contiguous(), *args[1:], d_out[:100].contiguous(), saved=True)
    layer.backward(*args, d_out, saved=True)
    layer.backward(*args, d_out)
    with pytest.raises(M.MoEError):
        layer.backward(*args, d_out, saved=True)
    # a layer without the backward workspace has no training forward
    plain = M.MoELayer.from_config(cfg)
    with pytest.raises(M.MoEError):
        plain.forward(*args, train=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["grouped", "stream"])
def test_layer_skewed_routing(path):
    """A +10 selection bias on experts 1, 2 (group 0) and 6 (group 1) sends
    every token to them: three experts with all 1100 rows each (five row
    tiles of 224, 224, 224, 224, 204 rows on the grouped path), the others
    empty."""
    inp = MI.make_layer(SKEWED, DEV)
    b = inp.sel_bias.clone()
    b[[1, 2, 6]] += 10.0
    inp = dataclasses.replace(inp, sel_bias=b)
    info, _ = _check_layer(inp, path=path)
    idx, _, counts = M.MoELayer.from_config(SKEWED).router(inp.x, inp.gate_w, inp.sel_bias)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    assert c[1] == c[2] == c[6] == SKEWED.T and c.sum() == 3 * SKEWED.T


DEGENERATE = MI.LayerConfig("every_kept_expert", T=600, D=256, E=16, H=128, G=4, kg=2, K=8, score_fn="softmax",
                            bias="none", norm=True, rsf=1.0, Hs=128, act="bf16", weight="bf16")


def test_layer_selects_every_expert_of_the_kept_groups():
    """K = kg*E/G: the selection is exactly the two kept groups' eight experts,
    so the group choice alone decides the routing; renormalised gates sum to 1."""
    inp = MI.make_layer(DEGENERATE, DEV)
    _check_layer(inp, path="grouped")
    idx, gate, _ = M.MoELayer.from_config(DEGENERATE).router(inp.x, inp.gate_w, None)
    torch.cuda.synchronize()
    groups = np.sort(idx.cpu().numpy() // (DEGENERATE.E // DEGENERATE.G), axis=1)
    assert np.all(groups[:, :4] == groups[:, :1]) and np.all(groups[:, 4:] == groups[:, 4:5])
    assert np.allclose(gate.sum(dim=1).cpu().numpy(), 1.0, atol=1e-5)


def test_bias_update_and_load_stats_match_the_oracle():
    """Bit-exact bias update (integer over/underload decision, fp32 sums) and
    load statistics within 1e-6 relative, for E from 1 to 512, with experts
    exactly at the mean load and with no assignments at all."""
    rng = np.random.default_rng(11)
    for E in (1, 12, 64, 256, 512):
        # counts = mean + d with sum(d) = 0, d = 0 on the first E/8 experts
        d = rng.integers(-30, 31, size=E)
        tied = max(1, E // 8)
        d[:tied] = 0
        if E > tied:
            rest = -int(d.sum())
            d[tied:] += rest // (E - tied)
            d[tied:tied + rest % (E - tied)] += 1
        counts = (1000 + d).astype(np.int32)
        assert counts.sum() == 1000 * E and np.all(counts[:tied] == 1000)
        for cnt in (counts, np.zeros(E, dtype=np.int32)):
            bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
            b = torch.tensor(bias, device=DEV)
            c = torch.tensor(cnt, device=DEV)
            M.bias_update(c, b, 1e-3)
            st = M.load_stats(c).cpu().numpy()
            torch.cuda.synchronize()
            assert np.array_equal(b.cpu().numpy(), O.bias_update(cnt, bias, 1e-3)), E
            ref = O.load_stats(cnt)
            for i, k in enumerate(("load_std", "load_loss", "max_violation")):
                assert abs(st[i] - ref[k]) <= 1e-6 * max(1.0, abs(ref[k])), (E, k, st[i], ref[k])


def test_bias_update_closes_the_loop_on_the_gpu():
    """Route, count, update the bias, repeat: each update equals the oracle's
    update of the GPU's own counts, and the skewed load evens out."""
    cfg = SMALL_SIG
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg)
    bias = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
    bias[:4] = 0.3
    std0 = None
    for step in range(40):
        _, _, counts = layer.router(inp.x, inp.gate_w, bias)
        before = bias.cpu().numpy()
        M.bias_update(counts, bias, 0.01)
        torch.cuda.synchronize()
        cnt = counts.cpu().numpy()
        assert np.array_equal(bias.cpu().numpy(), O.bias_update(cnt, before, 0.01)), step
        if std0 is None:
            std0 = O.load_stats(cnt)["load_std"]
    _, _, counts = layer.router(inp.x, inp.gate_w, bias)
    std = float(M.load_stats(counts)[0])
    assert std < 0.5 * std0, (std, std0)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[name] = MI.make_layer(MI.CONFIGS[name], DEV)
        return cache[name]
    yield get
    cache.clear()
    torch.cuda.empty_cache()


def test_layer_tiny_f32(layers):
    _check_layer(layers("tiny_f32"))


def test_layer_group_bf16(layers):
    inp = layers("group_bf16")
    _check_layer(inp, path="grouped")
    _check_layer(inp, tokens=_sample(inp.cfg.T, 256), path="stream", compose=True)


def _check_full_size(inp, n_random):
    """Outputs on every expert's first and last token plus n_random seeded
    tokens, for the full layer and a routed-only run."""
    R = A.route_inputs(inp)
    tokens = _cover_experts(R, inp.cfg.E, n_random)
    return _check_layer(inp, tokens=tokens, compose=True, R=R)


@pytest.mark.timeout(900)
def test_layer_v2_prefill(layers):
    _check_full_size(layers("v2_prefill"), 48)


@pytest.mark.timeout(900)
def test_layer_v3_prefill(layers):
    _check_full_size(layers("v3_prefill"), 24)


@pytest.mark.timeout(900)
def test_layer_v3_ep8_shard(layers):
    _check_full_size(layers("v3_ep8_shard"), 16)


@pytest.mark.timeout(900)
def test_layer_v3_prefill_w8a8(layers):
    """The V3 prefill layer with e4m3 activations, at full size; the
    quantiser bit for bit on sampled token rows of the same x."""
    inp = layers("v3_prefill_w8a8")
    _quant_parity(inp.x.cpu(), rows=_sample(inp.cfg.T, 64, seed=3))
    _check_full_size(inp, 16)


@pytest.mark.timeout(900)
def test_training_step_v3_prefill(layers):
    """The training forward and the saved backward at the V3 prefill shape,
    bit for bit against the grouped forward and the recomputing backward."""
    _train_step_matches(MI.CONFIGS["v3_prefill"], layers("v3_prefill"))
    torch.cuda.empty_cache()


def test_backward_v3_prefill_sampled(layers):
    """The backward pass at the V3 prefill shape: dx on sampled tokens and the
    weight gradients of two experts (all their tokens), against the oracle on
    the GPU's own expert choice (near-tie tokens may pick either side)."""
    inp = layers("v3_prefill")
    cfg = inp.cfg
    layer = M.MoELayer.from_config(cfg, backward=True)
    d_out = torch.randn((cfg.T, cfg.D), generator=torch.Generator().manual_seed(8)).to(DEV)
    got = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out)
    idx, _, _ = layer.router(inp.x, inp.gate_w, inp.sel_bias)
    torch.cuda.synchronize()
    R = A.route_inputs(inp)
    near = near_tie_mask(R)
    gidx = idx.cpu().numpy().astype(np.int64)
    R = dict(R)
    R["idx"] = np.where(near[:, None], gidx, R["idx"])
    R["gate"] = O.gate_values(R["scores"], R["idx"], cfg.norm, cfg.rsf)
    tokens = _sample(cfg.T, 12, seed=4)
    tokens = tokens[~near[tokens]]
    load = np.bincount(R["idx"].ravel(), minlength=cfg.E)
    experts = [int(np.argmax(load)), int(np.argmin(np.where(load > 0, load, 1 << 30)))]
    ref = O.layer_backward_sample(A.router_params(cfg), A.decode_tensor(inp.x), A.decode_tensor(inp.gate_w),
                                  A.routed_expert_fn(inp.experts), d_out.cpu().numpy().astype(np.float64), R,
                                  tokens, experts, A.shared_expert_fn(inp.shared), add_residual=cfg.add_residual)
    dx = got["dx"][torch.as_tensor(tokens, device=DEV)].cpu().numpy().astype(np.float64)
    e_dx = float((np.abs(dx - ref["dx"]).max(axis=1) / np.abs(ref["dx"]).max(axis=1)).max())
    e_w = 0.0
    for e in experts:
        dwg, dwu, dwd = ref["d_routed"][e]
        e_w = max(e_w, _rel_rows(got["d_gate_up"][e], np.concatenate([dwg, dwu], 0)), _rel_rows(got["d_down"][e], dwd))
    print(f"v3 backward: dx err {e_dx} over {len(tokens)} tokens, expert grads err {e_w} "
          f"(experts {experts}, rows {load[experts].tolist()}), near-tie tokens {int(near.sum())}")
    assert e_dx <= TOL["bf16"] and e_w <= TOL["bf16"]
    del got
    torch.cuda.empty_cache()


def test_layer_v3_decode_fp8(layers):
    inp = layers("v3_decode_fp8")
    _check_layer(inp)


def test_debug_build_matches_and_reports_no_violation():
    """The bounds-checked debug library gives bit-identical results on every
    kernel family (grouped and streaming bf16, e4m3 weights, e4m3
    activations, fp32, the backward pass, the training forward and the saved
    backward) and records no out-of-range index."""
    from mixture_experts_layer_38_amd import _binding as B
    from mixture_experts_layer_38_amd import build as Bd

    cases = [(SMALL_SIG, "grouped"), (SMALL_SIG, "stream"), (SMALL_FP8, "stream"), (SMALL_FP8, "grouped"),
             (SMALL_W8A8, "auto"), (SMALL_F32, "auto")]
    inputs = [MI.make_layer(c, DEV) for c, _ in cases]
    bw_inp = MI.make_layer(BWD_SIG, DEV)
    d_out = torch.randn((BWD_SIG.T, BWD_SIG.D), generator=torch.Generator().manual_seed(5)).to(DEV)

    def run_all():
        outs = []
        for (cfg, path), inp in zip(cases, inputs):
            layer = M.MoELayer.from_config(cfg, path=path)
            counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
            outs.append((layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared,
                                       expert_counts=counts), counts))
        layer = M.MoELayer.from_config(BWD_SIG, backward=True)
        g = layer.backward(bw_inp.x, bw_inp.gate_w, bw_inp.sel_bias, bw_inp.experts, bw_inp.shared, d_out)
        # the training forward (gate/up mode 3) and the backward that reads what it kept
        counts = torch.empty(BWD_SIG.E, dtype=torch.int32, device=DEV)
        outs.append((layer.forward(bw_inp.x, bw_inp.gate_w, bw_inp.sel_bias, bw_inp.experts, bw_inp.shared,
                                   expert_counts=counts, train=True), counts))
        g_saved = layer.backward(bw_inp.x, bw_inp.gate_w, bw_inp.sel_bias, bw_inp.experts, bw_inp.shared, d_out,
                                 saved=True)
        g.update({"saved_" + k: v for k, v in g_saved.items()})
        torch.cuda.synchronize()
        return outs, g

    ref_outs, ref_g = run_all()
    saved = (B.LIB_PATH, B._lib)
    try:
        B.LIB_PATH, B._lib = Bd.LIB_DEBUG, None
        B.load_library()
        assert M.debug_status() == (0, 0)
        outs, g = run_all()
        assert M.debug_status() == (0, 0)
    finally:
        B.LIB_PATH, B._lib = saved
    for (o, c), (ro, rc) in zip(outs, ref_outs):
        assert torch.equal(o, ro) and torch.equal(c, rc)
    for k in ("dx", "d_gate_w", "d_gate_up", "d_down", "saved_dx", "saved_d_gate_w", "saved_d_gate_up",
              "saved_d_down"):
        assert torch.equal(g[k], ref_g[k]), k

def test_binding_rejects_mismatched_tensors():
    """The binding checks every tensor against the cfg before the library
    sees a bare pointer: wrong dtype, shape, device or layout raise."""
    cfg = SMALL_FP8
    inp = MI.make_layer(cfg, DEV)
    layer = M.MoELayer.from_config(cfg)
    good = dict(x=inp.x, gate_w=inp.gate_w, sel_bias=inp.sel_bias, experts=inp.experts, shared=inp.shared)
    T = cfg.T
    bad_cases = [
        dict(out=torch.empty((T, cfg.D), dtype=torch.bfloat16, device=DEV)),   # cfg output is fp32
        dict(out=torch.empty((T - 1, cfg.D), dtype=torch.float32, device=DEV)),
        dict(expert_counts=torch.empty((cfg.E,), dtype=torch.int64, device=DEV)),
        dict(gate_w=inp.gate_w.to(torch.bfloat16)),
        dict(gate_w=inp.gate_w[:, :-1]),
        dict(gate_w=inp.gate_w.cpu()),
        dict(sel_bias=inp.sel_bias[:-1]),
        dict(experts=dataclasses.replace(inp.experts, down=inp.experts.down.transpose(1, 2))),
        dict(experts=dataclasses.replace(inp.experts, gate_up_scale=None)),
        dict(shared=None),
        dict(shared=dataclasses.replace(inp.shared, gate_up=inp.shared.gate_up.to(torch.bfloat16))),
    ]
    for bad in bad_cases:
        kw = dict(good)
        extra = {k: bad.pop(k) for k in ("out", "expert_counts") if k in bad}
        kw.update(bad)
        with pytest.raises(ValueError):
            layer.forward(kw["x"], kw["gate_w"], kw["sel_bias"], kw["experts"], kw["shared"], **extra)
    with pytest.raises(ValueError):
        layer.router(inp.x, inp.gate_w.t(), inp.sel_bias)
    with pytest.raises(ValueError):
        layer.dispatch(torch.zeros((4, cfg.K), dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        M.bias_update(torch.zeros(cfg.E, dtype=torch.int32, device=DEV), torch.zeros(cfg.E + 1, device=DEV), 1e-3)
    # the good call still runs
    layer.forward(**good)
    torch.cuda.synchronize()


def test_score_sums_and_balance_stats_match_the_oracle():
    """Score column sums written by the forward (sigmoid with bias, and
    softmax with groups) within 1e-5 relative of the oracle's fp64 sums, bit
    identical on a repeat and on the router entry point, zero for T = 0; the
    balance statistics on the GPU's own counts and sums against the oracle's
    at 1e-6 relative, and on the oracle's counts and sums at 1e-4."""
    for cfg in (SMALL_SIG, BWD_GROUP):
        inp = MI.make_layer(cfg, DEV)
        layer = M.MoELayer.from_config(cfg)
        S = torch.full((cfg.E,), -1.0, device=DEV)
        layer.set_score_sums(S)
        counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, expert_counts=counts)
        torch.cuda.synchronize()
        s1 = S.clone()
        R = A.route_inputs(inp)
        ref = O.score_sums(R["scores"])
        got = s1.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - ref) / ref) <= 1e-5, np.max(np.abs(got - ref) / ref)
        S.fill_(-1.0)
        layer.router(inp.x, inp.gate_w, inp.sel_bias)
        torch.cuda.synchronize()
        assert torch.equal(S, s1)
        for nd in (1, 4, cfg.E):
            st = M.balance_stats(counts, S, n_devices=nd).cpu().numpy()
            mine = O.balance_stats(counts.cpu().numpy(), S.cpu().numpy(), n_devices=nd)
            full = O.balance_stats(R["counts"], ref, n_devices=nd)
            for i, k in enumerate(M.BALANCE_STATS):
                assert abs(st[i] - mine[k]) <= 1e-6 * max(abs(mine[k]), 1e-6), (cfg.name, nd, k, st[i], mine[k])
                if not near_tie_mask(R).any():  # else a near-tie token may move one count
                    assert abs(st[i] - full[k]) <= 1e-4 * max(abs(full[k]), 1e-6), (cfg.name, nd, k, st[i], full[k])
        layer.forward(inp.x[:0], inp.gate_w, inp.sel_bias, inp.experts, inp.shared)
        torch.cuda.synchronize()
        assert not S.any()
        assert not M.balance_stats(torch.zeros(cfg.E, dtype=torch.int32, device=DEV), S, 2).any()
        layer.set_score_sums(None)
    with pytest.raises(ValueError):
        M.balance_stats(counts, S[:-1])
    with pytest.raises(M.MoEError):
        M.balance_stats(counts, S, n_devices=5)  # does not divide E
