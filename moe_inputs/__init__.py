"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module only draws tensors: it holds no step of the layer's arithmetic
(no routing, no expert FFN, no combine), so that the CPU oracle and the HIP
path can both be fed from it without sharing any compute code.

Every element is a pure function of (seed, tensor id, element index):

* the bit source is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to
  ``key + (index + 1) * 0x9E3779B97F4A7C15``, evaluated in wrapping int64
  torch arithmetic, so CPU and GPU produce the same bits;
* uniforms U(-a, a) use 23 bits: ``v = 2m + 1 - 2^23`` is an odd integer held
  exactly in float32 and ``w = v * (a * 2^-23)`` is one IEEE float32 multiply,
  so the float32 value is identical on every device; it is then rounded to the
  storage dtype (bf16 round-to-nearest-even, or e4m3 with a 128x128 block
  scale);
* normals use Box-Muller on two 53-bit uniforms, in float64 on the CPU.

Distributions follow the workloads the pages describe (DeepSeek-V2 walkthrough
page, MoEGate code: gate weights drawn by kaiming_uniform_(a=sqrt(5)), i.e.
U(+-1/sqrt(fan_in)); the same law is used for every expert matrix):
x ~ N(0, 1); gate_w, W_gate, W_up ~ U(+-1/sqrt(D)); W_down ~ U(+-1/sqrt(H)).
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field, replace

import torch

# ----------------------------------------------------------------------------
# bit source
# ----------------------------------------------------------------------------


def _s64(v: int) -> int:
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= (1 << 63) else v


_GOLDEN = _s64(0x9E3779B97F4A7C15)
_MIX1 = _s64(0xBF58476D1CE4E5B9)
_MIX2 = _s64(0x94D049BB133111EB)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 values."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _MIX1
    z = (z ^ _srl(z, 27)) * _MIX2
    return z ^ _srl(z, 31)


def splitmix64_scalar(state: int) -> int:
    """Python-int SplitMix64 output for one state value (used to derive keys)."""
    z = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    return z ^ (z >> 31)


def stream_key(seed: int, tensor_id: int) -> int:
    return _s64(splitmix64_scalar(splitmix64_scalar(seed) ^ (tensor_id * 0xD1B54A32D192ED03)))


def raw_bits(key: int, start: int, n: int, device) -> torch.Tensor:
    """64 random bits (as int64) for element indices start .. start+n-1."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix(idx * _GOLDEN + key)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

_CHUNK = 1 << 26


def uniform_pm(key: int, start: int, shape, a: float, device) -> torch.Tensor:
    """float32 U(-a, a) for element indices [start, start + numel)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float32, device=device)
    scale = float(torch.tensor(a, dtype=torch.float32)) * 2.0 ** -23  # exact power-of-two scaling
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        m = _srl(raw_bits(key, start + c0, c1 - c0, device), 41)  # 23 bits
        v = (2 * m + 1 - (1 << 23)).to(torch.float32)  # odd integer, exact in float32
        out[c0:c1] = v * scale
    return out.view(*shape)


def normal(key: int, start: int, shape, device="cpu") -> torch.Tensor:
    """float64 N(0, 1) by Box-Muller (computed on the CPU, then moved)."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float64)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        b = raw_bits(key, 2 * (start + c0), 2 * (c1 - c0), "cpu")
        m = _srl(b, 11).to(torch.float64)
        u = (m + 0.5) * 2.0 ** -53
        u1, u2 = u[0::2], u[1::2]
        out[c0:c1] = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return out.view(*shape).to(device)


def permutation(key: int, n: int) -> torch.Tensor:
    """A seeded permutation of 0..n-1 (argsort of random bits; ties by index)."""
    b = raw_bits(key, 0, n, "cpu")
    return torch.argsort(_srl(b, 1), stable=True)


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
FP8_BLOCK = 128


def quantize_e4m3_blocks(w: torch.Tensor):
    """Quantise a float32 [..., R, C] matrix to OCP e4m3 with one float32 scale
    per 128x128 block: scale = amax / 448, q = e4m3_rne(clamp(w / scale)).

    Returns (q as uint8 [..., R, C], scale float32 [..., R/128, C/128]).
    """
    *lead, R, C = w.shape
    assert R % FP8_BLOCK == 0 and C % FP8_BLOCK == 0
    wb = w.reshape(*lead, R // FP8_BLOCK, FP8_BLOCK, C // FP8_BLOCK, FP8_BLOCK)
    amax = wb.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    q = (wb / scale.unsqueeze(-1).unsqueeze(-3)).clamp(-E4M3_MAX, E4M3_MAX)
    q = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, R, C)
    return q, scale


def to_storage(w32: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return w32
    if dtype == "bf16":
        return w32.to(torch.bfloat16)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int  # tokens
    D: int  # model dim
    E: int  # routed experts
    H: int  # routed expert hidden
    G: int  # expert groups (1 = greedy)
    kg: int  # groups kept per token
    K: int  # routed experts per token
    score_fn: str  # "softmax" | "sigmoid"
    bias: str  # "none" | "normal" | "zipf"
    norm: bool  # renormalise the top-K gates
    rsf: float  # routed scaling factor
    Hs: int  # fused shared hidden (0 = no shared expert)
    act: str  # "f32" | "bf16"
    weight: str  # "f32" | "bf16" | "fp8"
    out: str = "f32"
    add_residual: bool = True
    act_quant: bool = False  # expert GEMM inputs quantised to e4m3 per 1x128 block (fp8 weights)
    seed: int = 0
    bias_std: float = 0.01

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    # page-1-style tiny layer (12 routed experts, top-4, 2 shared fused as hidden 2*128)
    "tiny_f32": LayerConfig("tiny_f32", T=256, D=64, E=12, H=128, G=1, kg=1, K=4,
                            score_fn="softmax", bias="none", norm=False, rsf=1.0, Hs=256,
                            act="f32", weight="f32"),
    # group-limited layer, bf16
    "group_bf16": LayerConfig("group_bf16", T=4096, D=1024, E=64, H=512, G=8, kg=3, K=6,
                              score_fn="softmax", bias="none", norm=False, rsf=1.0, Hs=1024,
                              act="bf16", weight="bf16"),
    # DeepSeek-V2-shaped prefill layer
    "v2_prefill": LayerConfig("v2_prefill", T=8192, D=5120, E=160, H=1536, G=8, kg=3, K=6,
                              score_fn="softmax", bias="none", norm=False, rsf=16.0, Hs=3072,
                              act="bf16", weight="bf16"),
    # DeepSeek-V3-shaped prefill layer
    "v3_prefill": LayerConfig("v3_prefill", T=16384, D=7168, E=256, H=2048, G=8, kg=4, K=8,
                              score_fn="sigmoid", bias="normal", norm=True, rsf=2.5, Hs=2048,
                              act="bf16", weight="bf16"),
    # decode-shaped V3 layer, e4m3 weights with 128x128 block scales, Zipf-skewed load
    "v3_decode_fp8": LayerConfig("v3_decode_fp8", T=64, D=7168, E=256, H=2048, G=8, kg=4, K=8,
                                 score_fn="sigmoid", bias="zipf", norm=True, rsf=2.5, Hs=2048,
                                 act="bf16", weight="fp8"),
    # the V3 prefill layer with the decode layer's e4m3 weights (128x128 block scales)
    "v3_prefill_fp8": LayerConfig("v3_prefill_fp8", T=16384, D=7168, E=256, H=2048, G=8, kg=4, K=8,
                                  score_fn="sigmoid", bias="normal", norm=True, rsf=2.5, Hs=2048,
                                  act="bf16", weight="fp8"),
    # the same with the expert GEMMs' inputs (token rows and h) quantised to
    # e4m3 per 1x128 block, multiplied on the fp8 matrix cores
    "v3_prefill_w8a8": LayerConfig("v3_prefill_w8a8", T=16384, D=7168, E=256, H=2048, G=8, kg=4, K=8,
                                   score_fn="sigmoid", bias="normal", norm=True, rsf=2.5, Hs=2048,
                                   act="bf16", weight="fp8", act_quant=True),
    # one GPU's share of the V3 prefill layer under 8-way expert parallelism:
    # 32 local experts, each receiving ~16384*8*8/256 = 4096 rows, the shared
    # expert on the GPU's own 16384 tokens (local top-8 of 32 reproduces the
    # expert-GEMM shapes; the exchange itself is not part of this workload)
    "v3_ep8_shard": LayerConfig("v3_ep8_shard", T=16384, D=7168, E=32, H=2048, G=1, kg=1, K=8,
                                score_fn="sigmoid", bias="normal", norm=True, rsf=2.5, Hs=2048,
                                act="bf16", weight="bf16"),
}
# the five workloads; v3_ep8_shard (sharding design), v3_prefill_fp8 and v3_prefill_w8a8 are extra shapes
CONFIG_ORDER = ["tiny_f32", "group_bf16", "v2_prefill", "v3_prefill", "v3_decode_fp8"]

# tensor ids: one independent stream per tensor
TID_X, TID_GATE_W, TID_BIAS, TID_GATE_UP, TID_DOWN, TID_SH_GATE_UP, TID_SH_DOWN = 1, 2, 3, 4, 5, 6, 7
TID_CALIB_X, TID_ZIPF_RANK = 8, 9

ZIPF_BIAS_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                              "tests", "golden", "zipf_bias_v3_e256.txt")


def gen_x(cfg: LayerConfig, device="cpu", T: int | None = None, tid: int = TID_X) -> torch.Tensor:
    T = cfg.T if T is None else T
    x = normal(stream_key(cfg.seed, tid), 0, (T, cfg.D), "cpu")
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    return x.to(dt).to(device)


def gen_gate_w(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    return uniform_pm(stream_key(cfg.seed, TID_GATE_W), 0, (cfg.E, cfg.D), 1.0 / math.sqrt(cfg.D), device)


def load_zipf_bias(E: int) -> torch.Tensor:
    vals = []
    with open(ZIPF_BIAS_FILE) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float.fromhex(line.split()[0]) if line.startswith(("0x", "-0x")) else float(line.split()[0]))
    b = torch.tensor(vals, dtype=torch.float32)
    if b.numel() != E:
        raise ValueError(f"zipf bias file holds {b.numel()} values, need {E}")
    return b


def gen_bias(cfg: LayerConfig, device="cpu"):
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        b = normal(stream_key(cfg.seed, TID_BIAS), 0, (cfg.E,)) * cfg.bias_std
        return b.to(torch.float32).to(device)
    if cfg.bias == "zipf":
        return load_zipf_bias(cfg.E).to(device)
    raise ValueError(cfg.bias)


def gen_expert_f32(cfg: LayerConfig, e: int, device="cpu"):
    """float32 (W_gate|W_up [2H, D], W_down [D, H]) of routed expert e."""
    n1 = 2 * cfg.H * cfg.D
    n2 = cfg.D * cfg.H
    gu = uniform_pm(stream_key(cfg.seed, TID_GATE_UP), e * n1, (2 * cfg.H, cfg.D), 1.0 / math.sqrt(cfg.D), device)
    dn = uniform_pm(stream_key(cfg.seed, TID_DOWN), e * n2, (cfg.D, cfg.H), 1.0 / math.sqrt(cfg.H), device)
    return gu, dn


def gen_shared_f32(cfg: LayerConfig, device="cpu"):
    gu = uniform_pm(stream_key(cfg.seed, TID_SH_GATE_UP), 0, (2 * cfg.Hs, cfg.D), 1.0 / math.sqrt(cfg.D), device)
    dn = uniform_pm(stream_key(cfg.seed, TID_SH_DOWN), 0, (cfg.D, cfg.Hs), 1.0 / math.sqrt(cfg.Hs), device)
    return gu, dn


@dataclass
class Weights:
    """Weights of one expert set in nn.Linear layout, as the C ABI takes them.

    gate_up [.., 2H, D] (rows 0..H-1 = W_gate, H..2H-1 = W_up), down [.., D, H].
    For fp8: uint8 e4m3 codes plus float32 scales [.., 2H/128, D/128] and
    [.., D/128, H/128].
    """
    gate_up: torch.Tensor
    down: torch.Tensor
    gate_up_scale: torch.Tensor | None = None
    down_scale: torch.Tensor | None = None


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor
    gate_w: torch.Tensor
    sel_bias: torch.Tensor | None
    experts: Weights
    shared: Weights | None
    extra: dict = field(default_factory=dict)


def _store(gu32, dn32, dtype):
    if dtype == "fp8":
        q1, s1 = quantize_e4m3_blocks(gu32)
        q2, s2 = quantize_e4m3_blocks(dn32)
        return q1, q2, s1, s2
    return to_storage(gu32, dtype), to_storage(dn32, dtype), None, None


def make_layer(cfg: LayerConfig, device="cpu", progress=None) -> LayerInputs:
    """All inputs of one layer, resident on `device`; `progress(e)` (optional)
    is called after expert e's weights are written."""
    x = gen_x(cfg, device)
    gate_w = gen_gate_w(cfg, device)
    bias = gen_bias(cfg, device)
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[cfg.weight]
    gu = torch.empty((cfg.E, 2 * cfg.H, cfg.D), dtype=wdt, device=device)
    dn = torch.empty((cfg.E, cfg.D, cfg.H), dtype=wdt, device=device)
    gus = dns = None
    if cfg.weight == "fp8":
        gus = torch.empty((cfg.E, 2 * cfg.H // FP8_BLOCK, cfg.D // FP8_BLOCK), dtype=torch.float32, device=device)
        dns = torch.empty((cfg.E, cfg.D // FP8_BLOCK, cfg.H // FP8_BLOCK), dtype=torch.float32, device=device)
    for e in range(cfg.E):
        a, b, sa, sb = _store(*gen_expert_f32(cfg, e, device), cfg.weight)
        gu[e].copy_(a)
        dn[e].copy_(b)
        if sa is not None:
            gus[e].copy_(sa)
            dns[e].copy_(sb)
        if progress is not None:
            progress(e)
    experts = Weights(gu, dn, gus, dns)
    shared = None
    if cfg.Hs > 0:
        a, b, sa, sb = _store(*gen_shared_f32(cfg, device), cfg.weight)
        shared = Weights(a, b, sa, sb)
    return LayerInputs(cfg, x, gate_w, bias, experts, shared)
