"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: brute force
over subsets on tiny inputs, closed forms, special cases that reduce to a
dense FFN or to the dense softmax mixture, and library decoders for the
storage formats. A dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them (test_pins_catch_planted_bugs
plants such mistakes in a copy of the oracle and checks that they are caught).
"""
import dataclasses
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.decode_bf16(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # format facts: largest finite 448, smallest subnormal 2^-9
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_e4m3_block_dequant_uses_the_right_block():
    codes = np.full((256, 384), 0x38, dtype=np.uint8)  # e4m3 1.0
    scale = np.arange(6, dtype=np.float32).reshape(2, 3) + 1.0
    w = O.dequant_e4m3_blocks(codes, scale)
    for i in range(2):
        for j in range(3):
            assert np.all(w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] == scale[i, j])


# ----------------------------------------------------------------------------
# e4m3 activations, one scale per 1 x 128 block
# ----------------------------------------------------------------------------


def _torch_e4m3(v):
    """torch's own float32 -> float8_e4m3fn cast (round to nearest even)."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_e4m3_matches_torch_cast():
    table = O.decode_e4m3(np.arange(0x7F))  # 0 .. 448
    mids = (table[:-1] + table[1:]) / 2  # every tie between neighbouring values
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)
    parts = [table, mids, RNG.uniform(-448, 448, 20000), RNG.standard_normal(20000) * 2.0 ** -7,
             RNG.standard_normal(2000) * 2.0 ** -12, np.array([463.9])]
    v = np.concatenate([np.concatenate([x, -x]) for x in parts]).astype(np.float32)
    assert np.array_equal(O.encode_e4m3(v), _torch_e4m3(v))


def test_encode_e4m3_round_trips_every_finite_code_and_saturates():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(O.encode_e4m3(O.decode_e4m3(codes).astype(np.float32)), codes)
    v = np.array([448.0, 463.9, 1e30, -1e30, -0.0, -2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10], np.float32)
    # saturation (reading), signed zero, ties to the even code among subnormals
    assert O.encode_e4m3(v).tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x02]


def test_quantize_act_closed_forms():
    x = RNG.standard_normal((5, 384)).astype(np.float32)
    x[1, 128:256] = 0  # an all-zero block
    x[3, :128] *= np.float32(2.0 ** -14)  # a block mostly in the subnormal range of its scale
    codes, scale = O.quantize_act_1x128(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32 and scale.shape == (5, 3)
    for r in range(5):
        for b in range(3):
            blk = x[r, 128 * b:128 * (b + 1)]
            amax = np.abs(blk).max()
            if amax == 0:
                assert scale[r, b] == 1 and not codes[r, 128 * b:128 * (b + 1)].any()
                continue
            assert scale[r, b] == amax / np.float32(448)
            j = int(np.argmax(np.abs(blk)))
            assert codes[r, 128 * b + j] == (0xFE if blk[j] < 0 else 0x7E)  # the block maximum maps to 448
    # codes are torch's cast of value / scale
    q = (x.reshape(5, 3, 128) / scale[:, :, None]).astype(np.float32)
    assert np.array_equal(codes, _torch_e4m3(q).reshape(5, 384))
    # within half a quantum: 2^-4 relative in e4m3's normal range, 2^-10 * scale below it
    xh = O.dequant_act_1x128(codes, scale)
    sc = np.repeat(scale.astype(np.float64), 128, axis=1)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc) * (1 + 1e-6)
    assert np.all(np.abs(xh - x) <= bound)


def test_quantize_act_blocks_are_independent_and_scale_exactly():
    x = RNG.standard_normal((3, 256)).astype(np.float32)
    c0, s0 = O.quantize_act_1x128(x)
    y = x.copy()
    y[:, 128:] *= np.float32(32.0)  # exact
    c1, s1 = O.quantize_act_1x128(y)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1[:, 0], s0[:, 0]) and np.array_equal(s1[:, 1], s0[:, 1] * np.float32(32.0))
    e, se = O.quantize_act_1x128(np.zeros((0, 128), np.float32))
    assert e.shape == (0, 128) and se.shape == (0, 1)


def test_e4m3_act_ffn_within_the_quantisation_error():
    """Both GEMM inputs quantised: the FFN stays within a few e4m3 quanta of
    the exact one, even with blocks whose magnitudes differ by 10^3 (a scale
    applied to the wrong block would not)."""
    rng = np.random.default_rng(77)
    D, h = 256, 128
    u = rng.standard_normal((40, D))
    u[:, :128] *= 1000.0
    u = u.astype(np.float32).astype(np.float64)
    wg = rng.uniform(-1, 1, (h, D)) / math.sqrt(D) / 100
    wu = rng.uniform(-1, 1, (h, D)) / math.sqrt(D) / 100
    wd = rng.uniform(-1, 1, (D, h)) / math.sqrt(h)
    exact = O.swiglu_ffn(u, wg, wu, wd)
    quant = O.swiglu_ffn_e4m3_act(u, wg, wu, wd)
    rel = np.linalg.norm(quant - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 0.08  # quantisation error (about 4 % here), far above float rounding
    # the routed and shared FFNs of the layer take the quantised form
    p = O.RouterParams(E=4, K=2)
    gw = RNG.standard_normal((4, D))
    out, r = O.layer_forward(p, u, gw, None, lambda e: (wg, wu, wd), lambda: (wg, wu, wd),
                             add_residual=False, act_quant=True)
    assert np.allclose(out, quant * (1 + r["gate"].sum(axis=1, keepdims=True)), rtol=1e-12, atol=1e-12)


def test_e4m3_act_ffn_hand_worked_example():
    """Each quantisation step of the e4m3-activation FFN on its own, worked by
    hand (D = hidden = 128, one block each):

    * u = [448, 12.4, 0, ...]: the block maximum is 448, so the scale is 1,
      and 12.4 becomes the e4m3 value 12 (between 8 and 16 the format steps
      by 1); gate rows 0 and 1 read u[1], so both gate pre-activations are
      12, not 12.4;
    * up row 0 is 1/448 and up row 1 is 16.5/448^2 on u[0] = 448: up values
      1 and 16.5/448;
    * h = [s, s*16.5/448, 0, ...] with s = SiLU(12) = 12 / (1 + e^-12): the
      block maximum s maps to 448 (scale s/448), and h[1] / scale = 16.5
      becomes the e4m3 value 16 (between 16 and 32 the format steps by 2);
    * the down projection picks h[0] and h[1] into outputs 0 and 1.

    So out = [s, 16 s / 448, 0, ...] up to the float32 roundings of h and of
    the scales (a few 2^-24). Skipping the quantisation of u gives
    SiLU(12.4) in out[0] (3 % off); skipping that of h gives 16.5 s / 448 in
    out[1] (3 % off); rounding h to bfloat16 before quantising it gives 12.0
    in out[0] (5e-6 off)."""
    D = h = 128
    u = np.zeros((1, D))
    u[0, 0], u[0, 1] = 448.0, 12.4
    u = u.astype(np.float32).astype(np.float64)
    wg = np.zeros((h, D))
    wg[0, 1] = wg[1, 1] = 1.0
    wu = np.zeros((h, D))
    wu[0, 0] = 1.0 / 448.0
    wu[1, 0] = 16.5 / 448.0 ** 2
    wd = np.zeros((D, h))
    wd[0, 0] = wd[1, 1] = 1.0
    got = O.swiglu_ffn_e4m3_act(u, wg, wu, wd)[0]
    s = 12.0 / (1.0 + math.exp(-12.0))
    want = np.zeros(D)
    want[0], want[1] = s, 16.0 * s / 448.0
    assert np.allclose(got, want, rtol=1e-6, atol=0.0), (got[:2], want[:2])


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------


def test_logits_brute_force():
    u = RNG.standard_normal((5, 7))
    w = RNG.standard_normal((3, 7))
    got = O.router_logits(u, w)
    for t in range(5):
        for e in range(3):
            acc = 0.0
            for d in range(7):
                acc += u[t, d] * w[e, d]
            assert abs(got[t, e] - acc) < 1e-12


def test_softmax_rows_sum_to_one_and_match_torch():
    l = RNG.standard_normal((64, 12)) * 3
    s = O.affinity(l, "softmax")
    assert np.allclose(s.sum(1), 1.0, atol=1e-12, rtol=0)
    ref = torch.softmax(torch.from_numpy(l), dim=-1).numpy()
    assert np.allclose(s, ref, atol=1e-15, rtol=1e-13)
    # shift invariance and monotonicity
    assert np.allclose(O.affinity(l + 5.0, "softmax"), s, atol=1e-15)
    assert np.array_equal(np.argsort(l, axis=1), np.argsort(s, axis=1))


def test_sigmoid_closed_forms():
    l = np.array([[0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0]])
    s = O.affinity(l, "sigmoid")
    assert s[0, 0] == 0.5
    assert abs(s[0, 1] - 0.75) < 1e-15 and abs(s[0, 2] - 0.25) < 1e-15
    assert s[0, 3] == 1.0 and s[0, 4] == 0.0


def _brute_select(z_row, G, kg, K):
    """Exhaustive search: the kept groups are the kg-subset with the largest sum
    of group maxima (lexicographically smallest index tuple among equals); the
    experts are the K-subset of their members with the largest sum of z (same
    tie rule)."""
    E = len(z_row)
    gs = E // G
    members = list(range(E))
    if G > 1:
        m = [max(z_row[j * gs:(j + 1) * gs]) for j in range(G)]
        best = None
        for S in itertools.combinations(range(G), kg):
            key = (sum(m[j] for j in S), tuple(-j for j in S))
            if best is None or key > best[0]:
                best = (key, S)
        members = [e for j in best[1] for e in range(j * gs, (j + 1) * gs)]
    best = None
    for S in itertools.combinations(members, K):
        key = (sum(z_row[e] for e in S), tuple(-e for e in sorted(S)))
        if best is None or key > best[0]:
            best = (key, S)
    return set(best[1])


@pytest.mark.parametrize("E,G,kg,K", [(8, 1, 1, 3), (8, 4, 2, 3), (12, 3, 2, 4), (12, 4, 4, 2),
                                      (16, 4, 1, 4), (9, 3, 2, 6), (6, 1, 1, 6)])
def test_selection_matches_brute_force(E, G, kg, K):
    # values on a coarse grid so that exact ties happen often
    for trial in range(60):
        z = RNG.integers(0, 6, size=(1, E)).astype(np.float64) / 4.0
        if trial % 3 == 0:
            z = RNG.standard_normal((1, E))
        idx, _, _, _ = O.select_experts(z, G, kg, K)
        assert set(idx[0].tolist()) == _brute_select(list(z[0]), G, kg, K)
        # canonical order: descending z, then ascending index
        order = sorted(idx[0].tolist(), key=lambda e: (-z[0, e], e))
        assert idx[0].tolist() == order


def test_all_groups_kept_and_single_group_are_greedy():
    z = RNG.standard_normal((200, 16))
    greedy = O.select_experts(z, 1, 1, 4)[0]
    assert np.array_equal(O.select_experts(z, 4, 4, 4)[0], greedy)
    assert np.array_equal(O.select_experts(z, 8, 8, 4)[0], greedy)
    # greedy: the K largest, verified by a full sort
    for t in range(200):
        assert set(greedy[t]) == set(np.argsort(-z[t], kind="stable")[:4])


def test_all_ties_pick_lowest_groups_and_indices():
    p = O.RouterParams(E=16, K=3, G=4, kg=2, score_fn="softmax")
    r = O.route(np.zeros((3, 8)), RNG.standard_normal((16, 8)), None, p)
    assert np.all(r["idx"] == [0, 1, 2])
    assert np.all(r["kept_groups"] == [0, 1])
    assert np.allclose(r["gate"], 1.0 / 16)


def test_large_bias_forces_an_expert_and_constant_bias_is_inert():
    T, D, E = 50, 16, 16
    u = RNG.standard_normal((T, D))
    w = RNG.standard_normal((E, D)) * 0.3
    p = O.RouterParams(E=E, K=4, G=4, kg=2, score_fn="sigmoid", norm=True, rsf=2.5)
    b = RNG.standard_normal(E) * 0.01
    r0 = O.route(u, w, b, p)
    b2 = b.copy()
    b2[11] = 10.0
    r1 = O.route(u, w, b2, p)
    assert np.all(np.any(r1["idx"] == 11, axis=1))
    assert r1["counts"][11] == T
    r2 = O.route(u, w, b + 3.0, p)
    assert np.array_equal(r2["idx"], r0["idx"])
    assert np.allclose(r2["gate"], r0["gate"], rtol=0, atol=1e-15)


def test_never_outside_kept_groups():
    T, E, G, kg = 300, 32, 8, 3
    z = RNG.standard_normal((T, E))
    idx, _, _, kept = O.select_experts(z, G, kg, 5)
    assert np.all(np.isin(idx // (E // G), kept).reshape(T, -1).all(axis=1))
    # the kept groups hold the kg largest group maxima
    m = z.reshape(T, G, -1).max(2)
    for t in range(T):
        assert set(kept[t]) == set(np.argsort(-m[t], kind="stable")[:kg])


def test_exclusion_differs_from_zero_fill_when_scores_are_negative():
    # z <= 0 everywhere (negative bias): an excluded expert must still never win
    z = np.array([[-0.5, -0.4, -0.1, -0.2, -0.9, -0.8, -0.7, -0.6]])
    idx, _, _, kept = O.select_experts(z, 4, 1, 2)
    assert kept[0].tolist() == [1]  # group {2,3} has the largest max (-0.1)
    assert set(idx[0].tolist()) == {2, 3}


def test_gates_normalised_sum_to_rsf_and_come_from_unbiased_scores():
    T, D, E = 40, 8, 12
    u = RNG.standard_normal((T, D))
    w = RNG.standard_normal((E, D))
    for fn in ("softmax", "sigmoid"):
        p = O.RouterParams(E=E, K=4, G=3, kg=2, score_fn=fn, norm=True, rsf=2.5)
        b = RNG.standard_normal(E) * 0.05
        r = O.route(u, w, b, p)
        assert np.allclose(r["gate"].sum(1), 2.5, atol=1e-12, rtol=0)
        # recompute from the unbiased scores on the chosen set
        s = r["scores"]
        for t in range(T):
            sel = s[t, r["idx"][t]]
            assert np.allclose(r["gate"][t], 2.5 * sel / sel.sum(), atol=1e-15)
        pn = O.RouterParams(E=E, K=4, G=3, kg=2, score_fn=fn, norm=False, rsf=16.0)
        rn = O.route(u, w, b, pn)
        assert np.array_equal(rn["idx"], r["idx"])
        assert np.allclose(rn["gate"], 16.0 * np.take_along_axis(s, r["idx"], 1), atol=1e-14)


def test_counts_sum_and_bincount():
    z = RNG.standard_normal((500, 20))
    idx = O.select_experts(z, 4, 2, 3)[0]
    c = O.expert_counts(idx, 20)
    assert c.sum() == 500 * 3
    assert np.array_equal(c, np.bincount(idx.ravel(), minlength=20))


def test_gaps_measure_the_selection_boundary():
    z = np.array([[0.9, 0.5, 0.5 + 1e-9, 0.1]])
    idx, gap_k, gap_g, _ = O.select_experts(z, 1, 1, 2)
    assert set(idx[0]) == {0, 2}
    assert abs(gap_k[0] - 1e-9) < 1e-15 and gap_g[0] == np.inf
    z = np.array([[0.9, 0.1, 0.3, 0.3, 0.2, 0.25]])
    idx, gap_k, gap_g, kept = O.select_experts(z, 3, 2, 2)
    assert kept[0].tolist() == [0, 1] and abs(gap_g[0] - 0.05) < 1e-15


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 50.0, -50.0, -800.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(s[2] + math.exp(-1.0) / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(s[3] - 50.0) < 1e-12 and abs(s[4]) < 1e-19 and s[5] == 0.0


def test_swiglu_worked_example():
    # D=3, h=2, worked by hand: gate = [1, -2], up = [4, 0.5]
    u = np.array([[1.0, 2.0, -1.0]])
    w_gate = np.array([[1.0, 0.0, 0.0], [0.0, -1.0, 0.0]])
    w_up = np.array([[0.0, 2.0, 0.0], [0.0, 0.0, -0.5]])
    w_down = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, -3.0]])
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    s2 = -2.0 / (1.0 + math.exp(2.0))
    h = np.array([s1 * 4.0, s2 * 0.5])
    expect = np.array([h[0], h[1], 2 * h[0] - 3 * h[1]])
    got = O.swiglu_ffn(u, w_gate, w_up, w_down)[0]
    assert np.allclose(got, expect, atol=1e-15, rtol=0)


def test_fine_grained_split_identity():
    """An FFN of hidden m*h equals the sum of its m slices taken as experts."""
    D, h, m = 16, 8, 4
    u = RNG.standard_normal((10, D))
    Wg = RNG.standard_normal((m * h, D))
    Wu = RNG.standard_normal((m * h, D))
    Wd = RNG.standard_normal((D, m * h))
    dense = O.swiglu_ffn(u, Wg, Wu, Wd)
    parts = sum(O.swiglu_ffn(u, Wg[i * h:(i + 1) * h], Wu[i * h:(i + 1) * h], Wd[:, i * h:(i + 1) * h])
                for i in range(m))
    assert np.allclose(dense, parts, atol=1e-12)


def _rand_experts(E, D, h, scale=0.3):
    return [(RNG.standard_normal((h, D)) * scale, RNG.standard_normal((h, D)) * scale,
             RNG.standard_normal((D, h)) * scale) for _ in range(E)]


def test_shared_fusion_identity():
    """Two shared experts of hidden h equal one fused shared expert of hidden 2h."""
    D, h, E = 12, 6, 6
    u = RNG.standard_normal((20, D))
    gw = RNG.standard_normal((E, D))
    p = O.RouterParams(E=E, K=2)
    ex = _rand_experts(E, D, h)
    s1, s2 = _rand_experts(2, D, h)
    fused = (np.vstack([s1[0], s2[0]]), np.vstack([s1[1], s2[1]]), np.hstack([s1[2], s2[2]]))
    out_f, r = O.layer_forward(p, u, gw, None, lambda e: ex[e], lambda: fused)
    out_0, _ = O.layer_forward(p, u, gw, None, lambda e: ex[e], None)
    assert np.allclose(out_f - out_0, O.swiglu_ffn(u, *s1) + O.swiglu_ffn(u, *s2), atol=1e-12)


def test_identical_experts_reduce_to_dense_ffn():
    D, h, E = 16, 8, 16
    u = RNG.standard_normal((30, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(1, D, h)[0]
    p = O.RouterParams(E=E, K=4, G=4, kg=2, score_fn="sigmoid", norm=True, rsf=2.5)
    b = RNG.standard_normal(E) * 0.01
    out, _ = O.layer_forward(p, u, gw, b, lambda e: ex, None, add_residual=False)
    assert np.allclose(out, 2.5 * O.swiglu_ffn(u, *ex), atol=1e-12)


def test_all_experts_softmax_is_the_dense_mixture():
    """K = E, one group, softmax, rsf 1: out = sum_e p_e FFN_e(u) (the dense
    einsum gate fusion of the architecture article, section 3.3)."""
    D, h, E = 8, 4, 6
    u = RNG.standard_normal((12, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(E, D, h)
    p = O.RouterParams(E=E, K=E)
    out, _ = O.layer_forward(p, u, gw, None, lambda e: ex[e], None, add_residual=False)
    ut = torch.from_numpy(u)
    probs = torch.softmax(ut @ torch.from_numpy(gw).T, dim=-1)
    outs = torch.stack([torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(ut, torch.from_numpy(g))) *
        torch.nn.functional.linear(ut, torch.from_numpy(up)), torch.from_numpy(dn)) for g, up, dn in ex], dim=1)
    dense = torch.einsum("ted,te->td", outs, probs).numpy()
    assert np.allclose(out, dense, atol=1e-12)


def test_top1_moe_without_shared_or_residual():
    D, h, E = 8, 4, 5
    u = RNG.standard_normal((25, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(E, D, h)
    p = O.RouterParams(E=E, K=1)
    out, r = O.layer_forward(p, u, gw, None, lambda e: ex[e], None, add_residual=False)
    l = u @ gw.T
    for t in range(25):
        e = int(np.argmax(l[t]))
        pmax = np.exp(l[t, e]) / np.exp(l[t]).sum()
        assert np.allclose(out[t], pmax * O.swiglu_ffn(u[t:t + 1], *ex[e])[0], atol=1e-12)


def test_residual_term_and_token_subset():
    D, h, E = 8, 4, 8
    u = RNG.standard_normal((20, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(E, D, h)
    sh = _rand_experts(1, D, 2 * h)[0]
    p = O.RouterParams(E=E, K=3, G=2, kg=1)
    o1, _ = O.layer_forward(p, u, gw, None, lambda e: ex[e], lambda: sh, add_residual=True)
    o0, _ = O.layer_forward(p, u, gw, None, lambda e: ex[e], lambda: sh, add_residual=False)
    assert np.allclose(o1 - o0, u, atol=1e-14)
    tok = np.array([7, 3, 19])
    os_, _ = O.layer_forward(p, u, gw, None, lambda e: ex[e], lambda: sh, tokens=tok)
    assert np.allclose(os_, o1[tok], atol=1e-14)


def test_permutation_equivariance():
    D, h, E = 8, 4, 8
    u = RNG.standard_normal((30, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(E, D, h)
    p = O.RouterParams(E=E, K=3)
    out, r = O.layer_forward(p, u, gw, None, lambda e: ex[e], None)
    tp = RNG.permutation(30)
    out_t, _ = O.layer_forward(p, u[tp], gw, None, lambda e: ex[e], None)
    assert np.allclose(out_t, out[tp], atol=1e-13)
    ep = RNG.permutation(E)  # expert j of the new layer is expert ep[j] of the old
    out_e, r_e = O.layer_forward(p, u, gw[ep], None, lambda e: ex[ep[e]], None)
    assert np.allclose(out_e, out, atol=1e-13)
    assert np.array_equal(np.sort(ep[r_e["idx"]], 1), np.sort(r["idx"], 1))


# ----------------------------------------------------------------------------
# load balance between steps
# ----------------------------------------------------------------------------


def test_bias_update_rule_closed_forms():
    """DeepSeek-V3 basics page, section 1.2: overloaded experts go down by
    gamma, underloaded ones up, and an expert exactly at the mean load stays."""
    b = np.array([0.5, -0.25, 0.0, 1.0], dtype=np.float32)
    out = O.bias_update([5, 1, 3, 3], b, 0.125)  # mean load 3
    assert out.dtype == np.float32
    assert out.tolist() == [0.375, -0.125, 0.0, 1.0]
    assert O.bias_update([2, 2, 2, 2], b, 0.125).tolist() == b.tolist()  # balanced: no change
    assert O.bias_update([0, 0, 0, 0], b, 0.125).tolist() == b.tolist()  # nothing routed
    # the new value is the float32 rounding of the exact sum
    one = np.array([1.0], dtype=np.float32)
    assert O.bias_update([0], one, 1e-8).tolist() == [1.0]
    assert O.bias_update([1, 0], np.float32([1.0, 1.0]), 2.0 ** -20).tolist() == [1.0 - 2.0 ** -20, 1.0 + 2.0 ** -20]


def test_bias_update_balances_a_skewed_router():
    """Applied step after step with the oracle router, the rule removes most
    of the imbalance that a skewed initial bias causes (its purpose in
    section 1.2), and the gates stay those of the unbiased scores."""
    T, D, E, K = 512, 32, 16, 2
    u = RNG.standard_normal((T, D))
    gw = RNG.standard_normal((E, D)) / math.sqrt(D)
    p = O.RouterParams(E=E, K=K, G=4, kg=2, score_fn="sigmoid", norm=True, rsf=1.0)
    b = np.zeros(E, dtype=np.float32)
    b[:3] = 0.3  # three experts favoured
    std0 = O.load_stats(O.route(u, gw, b.astype(np.float64), p)["counts"])["load_std"]
    for _ in range(60):
        R = O.route(u, gw, b.astype(np.float64), p)
        b = O.bias_update(R["counts"], b, 0.01)
    R = O.route(u, gw, b.astype(np.float64), p)
    assert O.load_stats(R["counts"])["load_std"] < 0.35 * std0
    s = O.affinity(O.router_logits(u, gw), "sigmoid")
    g = np.take_along_axis(s, R["idx"], 1)
    assert np.allclose(R["gate"], g / g.sum(1, keepdims=True), atol=1e-12)


def test_load_stats_closed_forms():
    E = 8
    z = O.load_stats(np.full(E, 5))
    assert z == {"load_std": 0.0, "load_loss": 0.0, "max_violation": 0.0}
    one = O.load_stats(np.eye(E, dtype=np.int64)[3] * 40)  # every assignment on one expert
    assert math.isclose(one["load_std"], 1 / math.sqrt(E), rel_tol=1e-12)
    assert math.isclose(one["load_loss"], (E - 1) / E ** 2, rel_tol=1e-12)
    assert math.isclose(one["max_violation"], E - 1, rel_tol=1e-12)
    assert O.load_stats(np.zeros(E, dtype=np.int64)) == {"load_std": 0.0, "load_loss": 0.0, "max_violation": 0.0}
    c = RNG.integers(0, 50, size=64)
    st = O.load_stats(c)
    load = torch.tensor(c, dtype=torch.float64) / c.sum()
    assert math.isclose(st["load_std"], float(load.std()), rel_tol=1e-12)  # torch's n-1 std
    assert math.isclose(st["max_violation"], c.max() * 64 / c.sum() - 1, rel_tol=1e-12)


def test_balance_stats_closed_forms():
    """Expert- and device-level balance statistics (load and importance) on
    cases worked by hand."""
    E = 8
    z = O.balance_stats(np.full(E, 5), np.full(E, 2.5), n_devices=4)
    assert all(v == 0.0 for v in z.values()), z
    # every assignment and all the score mass on expert 3 (device 1 of 4)
    one = O.balance_stats(np.eye(E, dtype=np.int64)[3] * 40, np.eye(E)[3] * 7.0, n_devices=4)
    for name in ("load", "importance"):
        assert math.isclose(one[f"{name}_std"], 1 / math.sqrt(E), rel_tol=1e-12)
        assert math.isclose(one[f"{name}_loss"], (E - 1) / E ** 2, rel_tol=1e-12)
        assert math.isclose(one[f"device_{name}_std"], 1 / math.sqrt(4), rel_tol=1e-12)
        assert math.isclose(one[f"device_{name}_loss"], 3 / 16, rel_tol=1e-12)
    assert math.isclose(one["max_violation"], E - 1, rel_tol=1e-12)
    # half the experts at twice the mean, half empty: deviations +-1/E
    half = O.balance_stats(np.array([2, 2, 2, 2, 0, 0, 0, 0]) * 9, np.array([2, 0] * 4, np.float64), n_devices=2)
    assert math.isclose(half["load_std"], math.sqrt(1 / (E * (E - 1))), rel_tol=1e-12)
    assert math.isclose(half["load_loss"], 1 / E ** 2, rel_tol=1e-12)
    assert math.isclose(half["importance_loss"], 1 / E ** 2, rel_tol=1e-12)
    # devices own contiguous runs: the load sits on device 0 ([1, 0]), while
    # the importance alternates and is even across the two devices
    assert math.isclose(half["device_load_std"], math.sqrt(0.5), rel_tol=1e-12)
    assert math.isclose(half["device_load_loss"], 0.25, rel_tol=1e-12)
    assert half["device_importance_std"] == 0.0 and half["device_importance_loss"] == 0.0
    # empty batch: all zero; one device: device statistics zero; E devices: the expert ones
    assert all(v == 0.0 for v in O.balance_stats(np.zeros(E, np.int64), np.zeros(E)).values())
    c = RNG.integers(0, 50, size=64)
    S = RNG.random(64) * 30
    st1 = O.balance_stats(c, S, n_devices=1)
    assert st1["device_load_std"] == st1["device_load_loss"] == st1["device_importance_loss"] == 0.0
    stE = O.balance_stats(c, S, n_devices=64)
    for name in ("load", "importance"):
        assert math.isclose(stE[f"device_{name}_std"], stE[f"{name}_std"], rel_tol=1e-12)
        assert math.isclose(stE[f"device_{name}_loss"], stE[f"{name}_loss"], rel_tol=1e-12)
    # torch's n-1 std; scale invariance; the count statistics equal load_stats
    imp = torch.tensor(S, dtype=torch.float64) / S.sum()
    assert math.isclose(st1["importance_std"], float(imp.std()), rel_tol=1e-12)
    st3 = O.balance_stats(c * 3, S * 0.5, n_devices=1)
    assert all(math.isclose(st3[k], st1[k], rel_tol=1e-12, abs_tol=1e-15) for k in st1)
    ls = O.load_stats(c)
    assert all(math.isclose(st1[k], ls[k], rel_tol=1e-12) for k in ls)


def test_score_sums_of_softmax_add_up_to_the_tokens():
    """Softmax scores of each token sum to 1, so the column sums add up to T;
    a token's sigmoid scores each lie in (0, 1)."""
    u = RNG.standard_normal((37, 16))
    w = RNG.standard_normal((12, 16))
    S = O.score_sums(O.affinity(O.router_logits(u, w), "softmax"))
    assert math.isclose(S.sum(), 37.0, rel_tol=1e-12)
    S2 = O.score_sums(O.affinity(O.router_logits(u, w), "sigmoid"))
    assert np.all((S2 > 0) & (S2 < 37))
    one = O.score_sums(O.affinity(O.router_logits(u[:1], w), "sigmoid"))
    assert np.allclose(one, 1 / (1 + np.exp(-(u[0] @ w.T))), rtol=1e-14)


# ----------------------------------------------------------------------------
# backward: the chain rule against central finite differences
# ----------------------------------------------------------------------------


def _bwd_problem(score_fn, norm, G, kg, seed, shared=True):
    """A small layer whose routing has no near-tie (every selection gap well
    above the finite-difference step), as float64 arrays."""
    T, D, E, h, K = 10, 12, 8, 6, 3
    for s in range(seed, seed + 200):
        rng = np.random.default_rng(s)
        u = rng.standard_normal((T, D))
        gw = rng.standard_normal((E, D)) / math.sqrt(D)
        bias = rng.standard_normal(E) * 0.05
        ex = {e: (rng.standard_normal((h, D)) / math.sqrt(D), rng.standard_normal((h, D)) / math.sqrt(D),
                  rng.standard_normal((D, h)) / math.sqrt(h)) for e in range(E)}
        sh = (rng.standard_normal((2 * h, D)) / math.sqrt(D), rng.standard_normal((2 * h, D)) / math.sqrt(D),
              rng.standard_normal((D, 2 * h)) / math.sqrt(2 * h)) if shared else None
        dout = rng.standard_normal((T, D))
        p = O.RouterParams(E=E, K=K, G=G, kg=kg, score_fn=score_fn, norm=norm, rsf=2.5)
        r = O.route(u, gw, bias, p)
        if min(r["gap_k"].min(), r["gap_g"].min()) > 1e-3:
            return p, u, gw, bias, ex, sh, dout
    raise AssertionError("no tie-free draw")


def _loss(p, u, gw, bias, ex, sh, dout):
    out, _ = O.layer_forward(p, u, gw, bias, lambda e: ex[e], (lambda: sh) if sh is not None else None)
    return float((dout * out).sum())


def _fd(f, arr, picks, eps=1e-6):
    g = []
    for ix in picks:
        old = arr[ix]
        arr[ix] = old + eps
        fp = f()
        arr[ix] = old - eps
        fm = f()
        arr[ix] = old
        g.append((fp - fm) / (2 * eps))
    return np.array(g)


@pytest.mark.parametrize("score_fn,norm,G,kg", [("sigmoid", True, 4, 2), ("softmax", False, 1, 1),
                                                ("softmax", True, 4, 3), ("sigmoid", False, 2, 1)])
def test_layer_backward_matches_finite_differences(score_fn, norm, G, kg):
    p, u, gw, bias, ex, sh, dout = _bwd_problem(score_fn, norm, G, kg, seed=3)
    g = O.layer_backward(p, u, gw, bias, lambda e: ex[e], dout, (lambda: sh))
    f = lambda: _loss(p, u, gw, bias, ex, sh, dout)  # noqa: E731
    rng = np.random.default_rng(0)

    def check(arr, grad, n=12):
        picks = [tuple(int(rng.integers(0, d)) for d in arr.shape) for _ in range(n)]
        num = _fd(f, arr, picks)
        ana = np.array([grad[ix] for ix in picks])
        scale = max(np.abs(ana).max(), 1e-3)
        assert np.abs(num - ana).max() <= 1e-6 * scale, (num, ana)

    check(u, g["dx"])
    check(gw, g["d_gate_w"])
    used = sorted(g["d_routed"])
    for e in used[:3]:
        for w, dw in zip(ex[e], g["d_routed"][e]):
            check(w, dw, n=6)
    for w, dw in zip(sh, g["d_shared"]):
        check(w, dw, n=6)
    # an expert nobody chose gets no gradient: the loss does not depend on it
    unused = [e for e in range(p.E) if e not in g["d_routed"]]
    for e in unused[:1]:
        assert np.all(_fd(f, ex[e][0], [(0, 0), (1, 2)]) == 0.0)
    # the selection bias only moves the choice: zero derivative
    assert np.all(np.abs(_fd(f, bias, [(0,), (3,), (5,)])) < 1e-9)


def test_sampled_backward_equals_the_full_one():
    p, u, gw, bias, ex, sh, dout = _bwd_problem("softmax", True, 4, 3, seed=21)
    full = O.layer_backward(p, u, gw, bias, lambda e: ex[e], dout, (lambda: sh))
    toks = np.array([0, 3, 7])
    used = sorted(full["d_routed"])[:2]
    smp = O.layer_backward_sample(p, u, gw, lambda e: ex[e], dout, full["routing"], toks, used, (lambda: sh))
    assert np.allclose(smp["dx"], full["dx"][toks], rtol=1e-12, atol=1e-12)
    for e in used:
        for a_, b_ in zip(smp["d_routed"][e], full["d_routed"][e]):
            assert np.allclose(a_, b_, rtol=1e-12, atol=1e-12)


def test_layer_backward_residual_and_routed_only():
    p, u, gw, bias, ex, sh, dout = _bwd_problem("sigmoid", True, 4, 2, seed=11, shared=False)
    g1 = O.layer_backward(p, u, gw, bias, lambda e: ex[e], dout, None, add_residual=True)
    g0 = O.layer_backward(p, u, gw, bias, lambda e: ex[e], dout, None, add_residual=False)
    assert np.allclose(g1["dx"] - g0["dx"], dout, rtol=0, atol=1e-12)  # the residual passes d_out through
    assert g1["d_shared"] is None
    # dL/dg is the expert output against d_out: recover it from the forward
    out_a, R = O.layer_forward(p, u, gw, bias, lambda e: ex[e], None, add_residual=False)
    t, k = 4, 1
    e = int(R["idx"][t, k])
    y = O.swiglu_ffn(u[t:t + 1], *ex[e])[0]
    assert math.isclose(g0["d_gate"][t, k], float(dout[t] @ y), rel_tol=1e-12)


# ----------------------------------------------------------------------------
# the pins must catch plausible mistakes
# ----------------------------------------------------------------------------


def test_pins_catch_planted_bugs(monkeypatch):
    """Plant typical mistakes in the oracle (on the CPU) and check that the
    pins above fail for each of them."""
    D, h, E = 16, 8, 16
    u = RNG.standard_normal((30, D))
    gw = RNG.standard_normal((E, D))
    ex = _rand_experts(1, D, h)[0]
    good = O.swiglu_ffn

    def swapped(uu, g, up, dn):  # gate and up exchanged
        return good(uu, up, g, dn)
    monkeypatch.setattr(O, "swiglu_ffn", swapped)
    with pytest.raises(AssertionError):
        test_swiglu_worked_example()
    monkeypatch.setattr(O, "swiglu_ffn", good)

    good_gate = O.gate_values
    monkeypatch.setattr(O, "gate_values", lambda s, idx, norm, rsf: np.take_along_axis(s, idx, 1) * rsf)
    p = O.RouterParams(E=E, K=4, G=4, kg=2, score_fn="sigmoid", norm=True, rsf=2.5)
    out, _ = O.layer_forward(p, u, gw, None, lambda e: ex, None, add_residual=False)
    assert not np.allclose(out, 2.5 * good(u, *ex), atol=1e-12)  # dropped renormalisation caught
    monkeypatch.setattr(O, "gate_values", good_gate)

    good_sel = O.select_experts

    def ascending(z, G, kg, K):  # sign error in the selection
        return good_sel(-z, G, kg, K)
    monkeypatch.setattr(O, "select_experts", ascending)
    with pytest.raises(AssertionError):
        test_top1_moe_without_shared_or_residual()
    monkeypatch.setattr(O, "select_experts", good_sel)

    good_bias = O.bias_update

    def flipped(counts, bias, gamma):  # overloaded experts pushed further up
        return good_bias(counts, bias, -gamma)
    monkeypatch.setattr(O, "bias_update", flipped)
    with pytest.raises(AssertionError):
        test_bias_update_rule_closed_forms()
    with pytest.raises(AssertionError):
        test_bias_update_balances_a_skewed_router()
    monkeypatch.setattr(O, "bias_update", good_bias)

    good_enc = O.encode_e4m3

    def ties_up(v):  # ties rounded away from zero instead of to even
        x = np.asarray(v, np.float32)
        return good_enc(x * np.float32(1 + 2.0 ** -20))
    monkeypatch.setattr(O, "encode_e4m3", ties_up)
    with pytest.raises(AssertionError):
        test_encode_e4m3_matches_torch_cast()
    monkeypatch.setattr(O, "encode_e4m3", good_enc)

    good_deq = O.dequant_act_1x128

    def reversed_blocks(codes, scales):  # block scales applied to the wrong blocks
        return good_deq(codes, np.asarray(scales)[:, ::-1])
    monkeypatch.setattr(O, "dequant_act_1x128", reversed_blocks)
    with pytest.raises(AssertionError):
        test_e4m3_act_ffn_within_the_quantisation_error()
    with pytest.raises(AssertionError):
        test_quantize_act_closed_forms()
    monkeypatch.setattr(O, "dequant_act_1x128", good_deq)

    good_q = O.quantize_act_1x128

    def off_by_one(values):  # scale from 447 instead of the format's largest value
        x = np.asarray(values, np.float32)
        codes, scale = good_q(x)
        n, C = x.shape
        amax = np.abs(x.reshape(n, C // 128, 128)).max(axis=2)
        s2 = np.where(amax > 0, amax / np.float32(447), np.float32(1)).astype(np.float32)
        return O.encode_e4m3((x.reshape(n, C // 128, 128) / s2[:, :, None]).astype(np.float32)).reshape(n, C), s2
    monkeypatch.setattr(O, "quantize_act_1x128", off_by_one)
    with pytest.raises(AssertionError):
        test_quantize_act_closed_forms()
    monkeypatch.setattr(O, "quantize_act_1x128", good_q)

    good_ffn8 = O.swiglu_ffn_e4m3_act

    def qdq(v):
        return O.dequant_act_1x128(*O.quantize_act_1x128(np.asarray(v).astype(np.float32)))

    def u_not_quantised(uu, g, up, dn):  # only h quantised
        hh = O.silu(uu @ g.T) * (uu @ up.T)
        return qdq(hh) @ dn.T

    def h_not_quantised(uu, g, up, dn):  # only u quantised
        uq = qdq(uu)
        return (O.silu(uq @ g.T) * (uq @ up.T)) @ dn.T

    def h_via_bf16(uu, g, up, dn):  # h rounded to bfloat16 before its quantisation
        uq = qdq(uu)
        hh = torch.from_numpy(O.silu(uq @ g.T) * (uq @ up.T)).to(torch.bfloat16).double().numpy()
        return qdq(hh) @ dn.T
    for bad in (u_not_quantised, h_not_quantised, h_via_bf16):
        monkeypatch.setattr(O, "swiglu_ffn_e4m3_act", bad)
        with pytest.raises(AssertionError):
            test_e4m3_act_ffn_hand_worked_example()
    monkeypatch.setattr(O, "swiglu_ffn_e4m3_act", good_ffn8)
    test_e4m3_act_ffn_hand_worked_example()

    good_bs = O.balance_stats

    def strided_devices(counts, score_sum, n_devices=1):  # device d owns experts e with e % n == d
        c = np.asarray(counts)
        S = np.asarray(score_sum, np.float64)
        E = c.shape[0]
        perm = np.arange(E).reshape(E // n_devices, n_devices).T.ravel()
        return good_bs(c[perm], S[perm], n_devices)

    def population_std(counts, score_sum, n_devices=1):  # n instead of n-1
        st = good_bs(counts, score_sum, n_devices)
        E = len(counts)
        for k in ("load_std", "importance_std"):
            st[k] *= math.sqrt((E - 1) / E)
        return st
    for bad in (strided_devices, population_std):
        monkeypatch.setattr(O, "balance_stats", bad)
        with pytest.raises(AssertionError):
            test_balance_stats_closed_forms()
    monkeypatch.setattr(O, "balance_stats", good_bs)

    good_sg = O.silu_grad
    monkeypatch.setattr(O, "silu_grad", lambda z: 1.0 / (1.0 + np.exp(-z)))  # sigma(z) for SiLU'(z)
    with pytest.raises(AssertionError):
        test_layer_backward_matches_finite_differences("sigmoid", True, 4, 2)
    monkeypatch.setattr(O, "silu_grad", good_sg)

    good_bwd = O.swiglu_ffn_backward

    def swapped_bwd(u, wg, wu, wd, dy):  # dW_gate and dW_up exchanged
        du, dwg, dwu, dwd, y = good_bwd(u, wg, wu, wd, dy)
        return du, dwu, dwg, dwd, y
    monkeypatch.setattr(O, "swiglu_ffn_backward", swapped_bwd)
    with pytest.raises(AssertionError):
        test_layer_backward_matches_finite_differences("softmax", False, 1, 1)
    monkeypatch.setattr(O, "swiglu_ffn_backward", good_bwd)

    good_gsg = O.gate_score_grad
    monkeypatch.setattr(O, "gate_score_grad", lambda s_sel, dg, norm, rsf: good_gsg(s_sel, dg, False, rsf))
    with pytest.raises(AssertionError):  # the renormalisation's coupling term dropped
        test_layer_backward_matches_finite_differences("sigmoid", True, 4, 2)
    monkeypatch.setattr(O, "gate_score_grad", good_gsg)
