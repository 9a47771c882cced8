"""Plain CPU oracle for the DeepSeekMoE layer forward, in float64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this
module: only the tests, the smoke check and the bench's CPU-baseline leg do.
It shares no code with the HIP library and takes plain numpy arrays.

What it computes, and where the pages define it (page titles as printed):

* "DeepSeek-V2 ... walkthrough" (page 1), section on the DeepSeekMoE
  architecture: the FFN output of token t is its input u_t plus the outputs of
  N_s always-active shared experts plus the gate-weighted outputs of the K_r
  routed experts with the highest token-to-expert affinity s_i,t. The same
  page's MoEGate code fixes the router: an fp32 linear map of the token to E
  logits, softmax scores, then greedy top-K or group-limited greedy top-K
  (per-group maximum, keep the best topk_group groups, top-K inside them).
  Its MoE code fuses the shared experts into one SwiGLU of hidden
  hidden_dim * n_shared_experts.
* "DeepSeekMoE + MLA" notes (page 3), section 2.1: p = softmax(W_gate x) and
  y = sum over the top-K of p_i E_i(x), gates not renormalised; section 5 and
  the architecture article (page 2, section 3.3): a SwiGLU expert without
  biases, down(SiLU(gate x) * up x).
* "DeepSeek-V3 basics" (page 5), section 1.2: a per-expert bias is added to
  the affinity only to choose the top-K; the gate value comes from the
  original affinity.
* "Transformer block" article (page 4), data-flow section: the scores may come
  from softmax or from another activation (sigmoid is used for the V3 shapes).
* "DeepSeek-V3 basics" (page 5), section 1.2, and the "DeepSeekMoE + MLA"
  notes (page 3), load-balance section: the bias update after a step and the
  load statistics (see bias_update and load_stats at the end).
* "Transformer block" article (page 4), training data-flow section, step 6:
  back-propagation updates the experts and the router; layer_backward gives
  those gradients by the chain rule through this forward.

Readings where the pages are silent or garbled (the formula images are
missing from the extracted pages):

* groups are contiguous runs of E/G experts (the view(n, n_group, -1) of the
  MoEGate code); the group score is the maximum of score + bias over the group;
* experts outside the kept groups are excluded outright (never selected);
* ties go to the lower group index and to the lower expert index; selected
  indices are listed by descending selection score, then ascending index;
* softmax is taken over all E logits before any masking;
* gates: g_k = s[idx_k]; if normalised, g_k /= sum_k s[idx_k]; then g_k *= rsf;
* the output includes the residual u_t when add_residual is set;
* e4m3 activations (architecture article, page 2, section 4.2, which fixes
  fp8 GEMM inputs, fp32 accumulation and block-wise quantisation but not the
  block shape): one fp32 scale per 1 x 128 block of a row, largest magnitude
  / 448, codes rounded to nearest-even, decided in float32.

Every routine below is pinned by tests in tests/test_oracle_pins.py (brute
force on tiny inputs, closed forms, reductions to a dense FFN or to the dense
softmax mixture, library decoders for the storage formats).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# storage formats: exact decoders
# ----------------------------------------------------------------------------


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16/int16) -> float64: the upper half of a
    float32, so widening by 16 zero bits is exact."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN codes stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_f32(values) -> np.ndarray:
    return np.asarray(values, dtype=np.float32).astype(np.float64)


def decode_e4m3(bits) -> np.ndarray:
    """OCP FP8 E4M3 codes -> float64, from the format's definition: 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (m/8 * 2^-6); S.1111.111 is NaN; no infinities; largest finite 448."""
    c = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0)
    sub = (man / 8.0) * 2.0 ** -6
    v = sign * np.where(ex == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


_E4M3_TABLE = None


def dequant_e4m3_blocks(codes, scale, block: int = 128) -> np.ndarray:
    """w[r, c] = e4m3(codes[r, c]) * scale[r // block, c // block] (the codes
    are decoded through a 256-entry table of decode_e4m3)."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = decode_e4m3(np.arange(256))
    c = np.asarray(codes)
    return apply_block_scales(_E4M3_TABLE[c.astype(np.intp)], scale, block)


def apply_block_scales(q, scale, block: int = 128) -> np.ndarray:
    """w[r, c] = q[r, c] * scale[r // block, c // block], in float64, for
    decoded e4m3 values q [..., R, C] and float32 scales [..., R/block, C/block]."""
    q = np.asarray(q, np.float64)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    *lead, R, C = q.shape
    qb = q.reshape(*lead, R // block, block, C // block, block)
    return (qb * s[..., :, None, :, None]).reshape(q.shape)


# ----------------------------------------------------------------------------
# e4m3 activations with one scale per 1 x 128 block
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
ACT_BLOCK = 128
_E4M3_MAGNITUDES = None  # values of codes 0x00 .. 0x7E, increasing


def encode_e4m3(values) -> np.ndarray:
    """float32 values -> OCP E4M3 codes: the representable value nearest to the
    value, ties to the even code (mantissa ending in 0). Readings: magnitudes
    above 448 saturate to 448; the sign bit is the float32 sign bit, so -0
    and negative values that round to zero give 0x80. Finite inputs only.
    Found by searching the 127 non-negative finite values of the format
    (decode_e4m3), not by bit manipulation."""
    global _E4M3_MAGNITUDES
    if _E4M3_MAGNITUDES is None:
        _E4M3_MAGNITUDES = decode_e4m3(np.arange(0x7F))
    table = _E4M3_MAGNITUDES
    x = np.asarray(values, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), E4M3_MAX)
    hi = np.minimum(np.searchsorted(table, a, side="left"), 0x7E)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quantize_act_1x128(values):
    """Fine-grained activation quantisation (the architecture article,
    section 4.2: fp8 inputs to the GEMMs, quantised block by block): each
    run of 128 consecutive elements of a row gets one fp32 scale, its largest
    magnitude divided by 448 (scale 1 for an all-zero block), and each element
    becomes the e4m3 code of value / scale. Both divisions are float32
    (correctly rounded), the precision the codes are decided in.
    values [n, C] (exact in float32), C % 128 == 0 -> (codes uint8 [n, C],
    scales float32 [n, C/128])."""
    x = np.asarray(values, dtype=np.float32)
    n, C = x.shape
    if C % ACT_BLOCK:
        raise ValueError("row length must be a multiple of 128")
    xb = x.reshape(n, C // ACT_BLOCK, ACT_BLOCK)
    amax = np.abs(xb).max(axis=2) if n else np.zeros((0, C // ACT_BLOCK), np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (xb / scale[:, :, None]).astype(np.float32)
    return encode_e4m3(q).reshape(n, C), scale


def dequant_act_1x128(codes, scales) -> np.ndarray:
    """x_hat[r, c] = e4m3(codes[r, c]) * scales[r, c // 128], in float64."""
    q = decode_e4m3(np.asarray(codes))
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    n, C = q.shape
    return (q.reshape(n, C // ACT_BLOCK, ACT_BLOCK) * s[:, :, None]).reshape(n, C)


# ----------------------------------------------------------------------------
# parameters
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class RouterParams:
    E: int  # routed experts
    K: int  # experts per token
    G: int = 1  # groups (1: greedy)
    kg: int = 1  # groups kept
    score_fn: str = "softmax"  # "softmax" | "sigmoid"
    norm: bool = False
    rsf: float = 1.0


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------


def router_logits(u: np.ndarray, gate_w: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_d u[t, d] * gate_w[e, d] (the MoEGate linear map, here in
    float64)."""
    return np.asarray(u, np.float64) @ np.asarray(gate_w, np.float64).T


def affinity(logits: np.ndarray, score_fn: str) -> np.ndarray:
    """s = softmax over all E experts, or the element-wise sigmoid."""
    if score_fn == "softmax":
        z = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(z)
        return ez / ez.sum(axis=1, keepdims=True)
    if score_fn == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-logits))
    raise ValueError(score_fn)


def select_experts(z: np.ndarray, G: int, kg: int, K: int):
    """Group-limited greedy top-K on selection scores z [T, E].

    Returns (idx [T, K] int64, gap_k [T], gap_g [T], kept_groups [T, kg]).
    gap_k is z_(K) - z_(K+1) over the candidate experts; gap_g is
    m_(kg) - m_(kg+1) over the group maxima (inf where no (K+1)-th exists).
    """
    T, E = z.shape
    rows = np.arange(T)
    allowed = np.ones((T, E), dtype=bool)
    gap_g = np.full(T, np.inf)
    kept = np.zeros((T, 0), dtype=np.int64)
    if G > 1:
        m = z.reshape(T, G, E // G).max(axis=2)
        gorder = np.argsort(-m, axis=1, kind="stable")  # descending, lower group first on ties
        kept = gorder[:, :kg]
        gmask = np.zeros((T, G), dtype=bool)
        gmask[rows[:, None], kept] = True
        allowed = np.repeat(gmask, E // G, axis=1)
        if kg < G:
            gap_g = m[rows, gorder[:, kg - 1]] - m[rows, gorder[:, kg]]
    zc = np.where(allowed, z, -np.inf)
    order = np.argsort(-zc, axis=1, kind="stable")  # descending, lower expert first on ties
    idx = order[:, :K]
    n_cand = int(allowed[0].sum()) if T else 0
    gap_k = np.full(T, np.inf)
    if n_cand > K:
        gap_k = zc[rows, order[:, K - 1]] - zc[rows, order[:, K]]
    return idx, gap_k, gap_g, kept


def gate_values(s: np.ndarray, idx: np.ndarray, norm: bool, rsf: float) -> np.ndarray:
    """g_k = s[idx_k] from the unbiased affinity; optional renormalisation over
    the K chosen experts; then the routed scaling factor."""
    g = np.take_along_axis(s, idx, axis=1)
    if norm:
        g = g / g.sum(axis=1, keepdims=True)
    return g * rsf


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """c[e] = number of (token, slot) pairs routed to expert e."""
    c = np.zeros(E, dtype=np.int64)
    for e in idx.reshape(-1):
        c[e] += 1
    return c


def route(u: np.ndarray, gate_w: np.ndarray, sel_bias, p: RouterParams) -> dict:
    logits = router_logits(u, gate_w)
    s = affinity(logits, p.score_fn)
    z = s if sel_bias is None else s + np.asarray(sel_bias, np.float64)[None, :]
    idx, gap_k, gap_g, kept = select_experts(z, p.G, p.kg, p.K)
    return dict(logits=logits, scores=s, z=z, idx=idx, gate=gate_values(s, idx, p.norm, p.rsf),
                counts=expert_counts(idx, p.E),
                gap_k=gap_k, gap_g=gap_g, kept_groups=kept)


# ----------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(u: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """FFN(u) = W_down (SiLU(W_gate u) * (W_up u)) for rows u [n, D]; weights in
    nn.Linear layout: w_gate, w_up [h, D], w_down [D, h]."""
    return (silu(u @ w_gate.T) * (u @ w_up.T)) @ w_down.T


def swiglu_ffn_e4m3_act(u: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """The same FFN with both GEMM inputs quantised to e4m3 per 1 x 128 block
    (architecture article, section 4.2): u is quantised before the gate and
    up projections; h = SiLU(gate) * up, rounded to float32 (the precision the
    kernel holds it in), is quantised before the down projection. The
    products and sums themselves are float64."""
    u = np.asarray(u, np.float64)
    if not np.array_equal(u.astype(np.float32).astype(np.float64), u):
        raise ValueError("inputs must be exact in float32")
    uq = dequant_act_1x128(*quantize_act_1x128(u.astype(np.float32)))
    h = silu(uq @ w_gate.T) * (uq @ w_up.T)
    hq = dequant_act_1x128(*quantize_act_1x128(h.astype(np.float32)))
    return hq @ w_down.T


def split_gate_up(gate_up: np.ndarray):
    """[2h, D] -> (W_gate = rows 0..h-1, W_up = rows h..2h-1)."""
    h = gate_up.shape[0] // 2
    return gate_up[:h], gate_up[h:]


def layer_forward(p: RouterParams, u: np.ndarray, gate_w: np.ndarray, sel_bias, routed_expert,
                  shared_expert=None, add_residual: bool = True, tokens=None, routing: dict | None = None,
                  act_quant: bool = False):
    """out_t = [u_t] + FFN_shared(u_t) + sum_k g_{t,k} FFN_{idx_{t,k}}(u_t).

    routed_expert(e) -> (w_gate, w_up, w_down) float64 for routed expert e;
    shared_expert() -> the same for the fused shared expert, or None.
    act_quant: every expert FFN (routed and shared) takes e4m3 activations
    (swiglu_ffn_e4m3_act); the router still sees u unquantised.
    Routing is computed for every token (counts need all of them); the
    output only for `tokens` (default: all), in that order.
    Returns (out [len(tokens), D], routing dict).
    """
    u = np.asarray(u, np.float64)
    if routing is None:
        routing = route(u, gate_w, sel_bias, p)
    T = u.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    ut = u[tokens]
    idx = routing["idx"][tokens]
    gate = routing["gate"][tokens]
    n, D = ut.shape
    # Y[i, k] = FFN_{idx[i, k]}(u_{tokens[i]}); each expert's weights are decoded once
    Y = np.zeros((n, p.K, D))
    ffn = swiglu_ffn_e4m3_act if act_quant else swiglu_ffn
    for e in np.unique(idx):
        ii, kk = np.nonzero(idx == e)
        Y[ii, kk] = ffn(ut[ii], *routed_expert(int(e)))
    out = np.zeros((n, D))
    if add_residual:
        out += ut
    if shared_expert is not None:
        sw = shared_expert()
        if sw is not None:
            out += ffn(ut, *sw)
    for k in range(p.K):
        out += gate[:, k:k + 1] * Y[:, k]
    return out, routing


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz SiLU(z) = sigma(z) (1 + z (1 - sigma(z)))."""
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu_ffn_backward(u, w_gate, w_up, w_down, dy):
    """Gradients of sum(dy * FFN(u)) for FFN(u) = W_down (SiLU(W_gate u) *
    (W_up u)): returns (du, dW_gate, dW_up, dW_down, y) with y = FFN(u)."""
    a = u @ w_gate.T
    b = u @ w_up.T
    sa = silu(a)
    h = sa * b
    y = h @ w_down.T
    dW_down = dy.T @ h
    dh = dy @ w_down
    da = dh * b * silu_grad(a)
    db = dh * sa
    return da @ w_gate + db @ w_up, da.T @ u, db.T @ u, dW_down, y


def gate_score_grad(s_sel: np.ndarray, d_gate: np.ndarray, norm: bool, rsf: float) -> np.ndarray:
    """dL/ds for the K selected scores from dL/dg, g_k = rsf * s_k (/ S with
    S = sum_j s_j when normalised): d g_k / d s_j = rsf (delta_jk / S - s_k / S^2)."""
    if not norm:
        return rsf * d_gate
    S = s_sel.sum(axis=1, keepdims=True)
    return rsf * (d_gate / S - (d_gate * s_sel).sum(axis=1, keepdims=True) / S ** 2)


def layer_backward(p: RouterParams, u: np.ndarray, gate_w: np.ndarray, sel_bias, routed_expert, d_out,
                   shared_expert=None, add_residual: bool = True, routing: dict | None = None):
    """Gradients of L = sum(d_out * out) for out = layer_forward(...), by the
    chain rule through the forward's definition. The expert choice (group
    limit and top-K) is piecewise constant, so it is held fixed and carries
    no gradient; the gradient reaches the router through the gate values
    g_k = rsf * s_k [/ sum_j s_j], then through the score function to the
    logits, x and gate_w. The selection bias changes only the choice, so it
    gets no gradient (the bias rule updates it between steps).

    Returns dict(dx [T, D], d_gate_w [E, D], d_routed {e: (dW_gate, dW_up,
    dW_down)} for every expert that received a token, d_shared (dW_gate,
    dW_up, dW_down) or None, d_gate [T, K] = dL/dg, routing)."""
    u = np.asarray(u, np.float64)
    d_out = np.asarray(d_out, np.float64)
    if routing is None:
        routing = route(u, gate_w, sel_bias, p)
    T, D = u.shape
    idx, gate, s = routing["idx"], routing["gate"], routing["scores"]
    dx = d_out.copy() if add_residual else np.zeros((T, D))
    d_gate = np.zeros((T, p.K))
    d_routed = {}
    for e in np.unique(idx):
        ii, kk = np.nonzero(idx == e)  # a token picks an expert at most once
        wg, wu, wd = routed_expert(int(e))
        dy = gate[ii, kk][:, None] * d_out[ii]
        du, dwg, dwu, dwd, y = swiglu_ffn_backward(u[ii], wg, wu, wd, dy)
        dx[ii] += du
        d_gate[ii, kk] = (d_out[ii] * y).sum(axis=1)
        d_routed[int(e)] = (dwg, dwu, dwd)
    d_shared = None
    if shared_expert is not None:
        sw = shared_expert()
        if sw is not None:
            du, dwg, dwu, dwd, _ = swiglu_ffn_backward(u, *sw, d_out)
            dx += du
            d_shared = (dwg, dwu, dwd)
    # gates -> selected scores -> all scores -> logits
    rows = np.arange(T)[:, None]
    ds_sel = gate_score_grad(s[rows, idx], d_gate, p.norm, p.rsf)
    ds = np.zeros_like(s)
    ds[rows, idx] = ds_sel
    if p.score_fn == "sigmoid":
        dlogit = ds * s * (1.0 - s)
    else:
        dlogit = s * (ds - (s * ds).sum(axis=1, keepdims=True))
    gw = np.asarray(gate_w, np.float64)
    dx += dlogit @ gw
    return dict(dx=dx, d_gate_w=dlogit.T @ u, d_routed=d_routed, d_shared=d_shared, d_gate=d_gate,
                routing=routing)


def layer_backward_sample(p: RouterParams, u: np.ndarray, gate_w: np.ndarray, routed_expert, d_out,
                          routing: dict, tokens, experts, shared_expert=None, add_residual: bool = True):
    """The same gradients as layer_backward, on a sample: dx for `tokens` and
    the weight gradients of the routed `experts` (from all their tokens).
    Each expert's and each token's share is computed on its own rows, with the
    same steps as layer_backward; d gate_w needs every token and is not
    returned. Returns dict(dx [len(tokens), D], d_routed {e: ...})."""
    u = np.asarray(u, np.float64)
    d_out = np.asarray(d_out, np.float64)
    tokens = np.asarray(tokens)
    idx, gate, s = routing["idx"], routing["gate"], routing["scores"]
    n, D = len(tokens), u.shape[1]
    dx = d_out[tokens].copy() if add_residual else np.zeros((n, D))
    d_gate = np.zeros((n, p.K))
    sel = idx[tokens]
    for e in np.unique(sel):  # each expert's weights decoded once
        jj, kk = np.nonzero(sel == e)
        tt = tokens[jj]
        wg, wu, wd = routed_expert(int(e))
        du, _, _, _, y = swiglu_ffn_backward(u[tt], wg, wu, wd, gate[tt, kk][:, None] * d_out[tt])
        dx[jj] += du
        d_gate[jj, kk] = (d_out[tt] * y).sum(axis=1)
    if shared_expert is not None:
        sw = shared_expert()
        if sw is not None:
            du, _, _, _, _ = swiglu_ffn_backward(u[tokens], *sw, d_out[tokens])
            dx += du
    rows = np.arange(n)[:, None]
    ds_sel = gate_score_grad(s[tokens][rows, idx[tokens]], d_gate, p.norm, p.rsf)
    ds = np.zeros((n, s.shape[1]))
    ds[rows, idx[tokens]] = ds_sel
    st = s[tokens]
    dlogit = ds * st * (1.0 - st) if p.score_fn == "sigmoid" else st * (ds - (st * ds).sum(axis=1, keepdims=True))
    dx += dlogit @ np.asarray(gate_w, np.float64)
    d_routed = {}
    for e in experts:
        ii, kk = np.nonzero(idx == e)
        wg, wu, wd = routed_expert(int(e))
        _, dwg, dwu, dwd, _ = swiglu_ffn_backward(u[ii], wg, wu, wd, gate[ii, kk][:, None] * d_out[ii])
        d_routed[int(e)] = (dwg, dwu, dwd)
    return dict(dx=dx, d_routed=d_routed)


def near_tie_tokens(routing: dict, window: float = 1e-6) -> np.ndarray:
    """Tokens whose K/K+1 or group-boundary selection-score gap is within the window."""
    return np.nonzero((routing["gap_k"] < window) | (routing["gap_g"] < window))[0]


# ----------------------------------------------------------------------------
# load balance between steps
# ----------------------------------------------------------------------------


def bias_update(counts, bias, gamma: float) -> np.ndarray:
    """Auxiliary-loss-free balancing ("DeepSeek-V3 basics", page 5, section
    1.2): after a step, an overloaded expert's selection bias goes down by
    gamma and an underloaded expert's goes up by gamma. Reading: overloaded
    means more assignments than the mean load sum(counts)/E, underloaded fewer;
    at exactly the mean the bias stays. The bias is stored as float32, so the
    new value is the float32 rounding of the exact sum."""
    c = np.asarray(counts, dtype=np.int64)
    E = c.shape[0]
    total = int(c.sum())
    b = np.asarray(bias, dtype=np.float32).astype(np.float64)
    out = b.copy()
    for e in range(E):
        if c[e] * E > total:
            out[e] = b[e] - float(np.float32(gamma))
        elif c[e] * E < total:
            out[e] = b[e] + float(np.float32(gamma))
    return out.astype(np.float32)


def load_stats(counts) -> dict:
    """Load statistics of one step ("DeepSeekMoE + MLA" notes, page 3, load
    balance code): load_e = counts_e / sum(counts); its standard deviation over
    the experts with the n-1 denominator (as torch's std), the load term
    mean_e (load_e - 1/E)^2 of the expert-level balance loss, and the maximum
    violation max_e counts_e / mean - 1 with mean = sum(counts) / E. With no
    assignments at all every statistic is 0."""
    c = np.asarray(counts, dtype=np.float64)
    E = c.shape[0]
    total = c.sum()
    if total == 0:  # no assignments: nothing is loaded (reading: all zero)
        return {"load_std": 0.0, "load_loss": 0.0, "max_violation": 0.0}
    load = c / total
    mean = total / E
    dev = load - load.mean()
    return {
        "load_std": float(np.sqrt((dev * dev).sum() / (E - 1))) if E > 1 else 0.0,
        "load_loss": float(((load - 1.0 / E) ** 2).mean()),
        "max_violation": float(c.max() / mean - 1.0),
    }


def score_sums(scores) -> np.ndarray:
    """S_e = sum over the tokens of s[t, e] (the column sums the importance
    statistic normalises), in float64."""
    return np.asarray(scores, np.float64).sum(axis=0)


def balance_stats(counts, score_sum, n_devices: int = 1) -> dict:
    """The statistics of the load-balance code in the "DeepSeekMoE + MLA"
    notes (page 3, expert- and device-level balance): load_e = c_e / sum(c)
    and importance_e = S_e / sum(S) (S the column sums of the scores); their
    standard deviations over the experts (n-1 denominator, as torch's std)
    and the loss terms mean((x - 1/E)^2); the same for devices, each owning a
    contiguous run of E / n_devices experts, whose load and importance are the
    sums over their experts renormalised to sum 1. Readings: the page's 1e-9
    in each denominator only guards an empty batch, so the normalisation is
    exact here and every statistic of a quantity whose total is 0 is 0; the
    standard deviation of a single value is 0. max_violation as in
    load_stats."""
    c = np.asarray(counts, dtype=np.float64)
    S = np.asarray(score_sum, dtype=np.float64)
    E = c.shape[0]
    if n_devices < 1 or E % n_devices:
        raise ValueError("n_devices must divide E")

    def spread(x):
        n = x.shape[0]
        std = float(np.sqrt(((x - x.mean()) ** 2).sum() / (n - 1))) if n > 1 else 0.0
        return std, float(((x - 1.0 / n) ** 2).mean())

    def normalise(x):
        return x / x.sum()

    out = {}
    for name, v in (("load", c), ("importance", S)):
        keys = (f"{name}_std", f"{name}_loss", f"device_{name}_std", f"device_{name}_loss")
        if v.sum() == 0:
            out.update({k: 0.0 for k in keys})
            continue
        x = normalise(v)
        dev = normalise(x.reshape(n_devices, E // n_devices).sum(axis=1))
        (out[keys[0]], out[keys[1]]), (out[keys[2]], out[keys[3]]) = spread(x), spread(dev)
    out["max_violation"] = float(c.max() / (c.sum() / E) - 1.0) if c.sum() > 0 else 0.0
    return out
