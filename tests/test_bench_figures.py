"""The bench's work and byte figures (the numerators of its rooflines) against
the workload definitions, computed here from the shapes term by term:
the V3 prefill layer's MFMA work and its gate/up launch, the algorithmic
bytes of that launch, and the fp8 decode layer's bytes per step for a given
number of touched experts. CPU only."""
import bench
import moe_inputs as MI

V3 = MI.CONFIGS["v3_prefill"]
DEC = MI.CONFIGS["v3_decode_fp8"]


def test_v3_prefill_mfma_work():
    # per routed (token, slot): gate, up and down products of D x H each, 2 flop
    # per multiply-add; the shared expert once per token with its own hidden size
    T, K, D, H, Hs = 16384, 8, 7168, 2048, 2048
    routed = T * K * 3 * (2 * D * H)
    shared = T * 3 * (2 * D * Hs)
    assert bench.mfma_flops(V3) == routed + shared == 12987981103104
    assert abs(bench.mfma_flops(V3) - 1.2988e13) / 1.2988e13 < 1e-4
    # the gate/up launch: two of the three products
    assert bench.gateup_flops(V3) == T * K * 2 * (2 * D * H) + T * 2 * (2 * D * Hs) == 8658654068736


def test_v3_prefill_gateup_algorithmic_bytes():
    T, K, D, H, Hs, E = 16384, 8, 7168, 2048, 2048, 256
    weights = 2 * (E * 2 * H + 2 * Hs) * D  # bf16 [2H][D] per routed expert and the shared one
    token_rows = 2 * (T * K + T) * D        # each gathered row once (routed slots and shared)
    h_out = 2 * (T * K * H + T * Hs)         # h written once
    assert bench.gateup_algorithmic_bytes(V3) == weights + token_rows + h_out


def test_v3_decode_bytes_per_step():
    T, D, H, Hs, E = 64, 7168, 2048, 2048, 256
    n = 125
    # e4m3 weights (one byte each) and one fp32 scale per 128 x 128 block
    expert = 3 * H * D + 4 * ((2 * H // 128) * (D // 128) + (D // 128) * (H // 128))
    shared = 3 * Hs * D + 4 * ((2 * Hs // 128) * (D // 128) + (D // 128) * (Hs // 128))
    assert expert == 44050944  # 44.05 MB per touched expert
    gate_w, bias = E * D * 4, E * 4
    x_in, out = T * D * 2, T * D * 4  # bf16 tokens in, fp32 output
    total, gate_up = bench.decode_bytes(DEC, n)
    assert total == n * expert + shared + gate_w + bias + x_in + out
    assert gate_w == 7340032 and x_in + out == 2752512
    # the gate/up launch streams two thirds of each touched expert's weights and the shared expert's
    gu_expert = 2 * H * D + 4 * (2 * H // 128) * (D // 128)
    gu_shared = 2 * Hs * D + 4 * (2 * Hs // 128) * (D // 128)
    assert gate_up == n * gu_expert + gu_shared
