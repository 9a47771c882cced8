"""The seeded input generator: determinism, independence of streams, the
distributions of the workloads, and the fp8 block-quantisation contract."""
import math

import numpy as np
import torch

import moe_inputs as MI
from oracle import moe_oracle as O


def test_splitmix64_published_vector():
    # first outputs of SplitMix64 seeded with 1234567 (reference implementation)
    b = MI.raw_bits(1234567, 0, 3, "cpu")
    assert [int(v) & ((1 << 64) - 1) for v in b] == [6457827717110365317, 3203168211198807973,
                                                     9817491932198370423]


def test_uniform_is_deterministic_sliceable_and_in_range():
    k = MI.stream_key(0, MI.TID_GATE_UP)
    a = MI.uniform_pm(k, 0, (1000, 64), 0.125, "cpu")
    b = MI.uniform_pm(k, 0, (1000, 64), 0.125, "cpu")
    assert torch.equal(a, b)
    c = MI.uniform_pm(k, 640, (10, 64), 0.125, "cpu")  # rows 10..19
    assert torch.equal(a[10:20], c)
    assert float(a.abs().max()) < 0.125
    assert abs(float(a.mean())) < 2e-3
    assert abs(float(a.var()) * 3 / 0.125 ** 2 - 1) < 0.02
    other = MI.uniform_pm(MI.stream_key(0, MI.TID_DOWN), 0, (1000, 64), 0.125, "cpu")
    assert abs(float(torch.corrcoef(torch.stack([a.ravel(), other.ravel()]))[0, 1])) < 0.02


def test_normal_moments():
    n = MI.normal(MI.stream_key(0, MI.TID_X), 0, (400000,))
    assert abs(float(n.mean())) < 0.01 and abs(float(n.std()) - 1) < 0.01
    assert abs(float((n ** 4).mean()) - 3) < 0.05  # normal kurtosis


def test_expert_generation_matches_whole_tensor_slices():
    cfg = MI.CONFIGS["tiny_f32"]
    inp = MI.make_layer(cfg)
    gu3, dn3 = MI.gen_expert_f32(cfg, 3)
    assert torch.equal(inp.experts.gate_up[3], gu3) and torch.equal(inp.experts.down[3], dn3)
    assert inp.x.shape == (256, 64) and inp.x.dtype == torch.float32
    assert inp.shared.gate_up.shape == (512, 64) and inp.shared.down.shape == (64, 256)
    assert float(inp.experts.down.abs().max()) < 1 / math.sqrt(128)


def test_fp8_block_quantisation_contract():
    w = MI.uniform_pm(MI.stream_key(5, 99), 0, (256, 384), 0.02, "cpu")
    q, s = MI.quantize_e4m3_blocks(w)
    assert q.dtype == torch.uint8 and s.shape == (2, 3)
    deq = O.dequant_e4m3_blocks(q.numpy(), s.numpy())
    # every block's largest magnitude maps to (about) 448 * scale, and the
    # quantisation error is within half an e4m3 step (2^-4 relative) plus subnormal spacing
    w64 = w.double().numpy()
    for i in range(2):
        for j in range(3):
            blk = np.abs(w64[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
            assert abs(blk.max() / s[i, j].item() - 448) < 1e-3
    err = np.abs(deq - w64)
    sfull = np.repeat(np.repeat(s.double().numpy(), 128, 0), 128, 1)
    assert np.all(err <= np.abs(w64) * 2.0 ** -4 + sfull * 2.0 ** -10)


def test_zipf_bias_file_and_config_table():
    b = MI.load_zipf_bias(256)
    assert b.dtype == torch.float32 and torch.isfinite(b).all()
    assert float(b.max() - b.min()) > 0.1  # a real skew
    cfgs = [MI.CONFIGS[n] for n in MI.CONFIG_ORDER]
    assert [c.T for c in cfgs] == [256, 4096, 8192, 16384, 64]
    assert [c.E for c in cfgs] == [12, 64, 160, 256, 256]
    assert [c.Hs for c in cfgs] == [256, 1024, 3072, 2048, 2048]
