"""Writes tests/golden/zipf_bias_v3_e256.txt: the per-expert selection bias of the
decode-shaped V3 workload (256 experts, 8 groups keep 4, top-8 sigmoid routing),
chosen so that expert popularity follows Zipf(s = 1.2).

The bias is found with the balancing rule of the "DeepSeek-V3 basics" page
(section 1.2, auxiliary-loss-free load balancing): after each step, an expert's
bias goes down by gamma if it is over its target load and up by gamma if under.
Here the target is a Zipf share instead of the uniform one:

1. a seeded permutation assigns ranks r_e in 1..256;
2. per-token selection probability p_e proportional to r_e^-1.2, scaled so that
   sum p_e = K and water-filled so that p_e <= 1;
3. on a calibration batch of 8192 tokens (its own input stream), starting from
   b = 0, repeat 300 times: route with the oracle router, then
   b_e += gamma * sign(p_e - load_e) (gamma = 1e-2 for 200 steps, then 1e-3).

Only the oracle and the seeded input generator are called. Run:
    python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_inputs as MI  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from oracle.adapter import decode_tensor  # noqa: E402

S_ZIPF = 1.2
CALIB_T = 8192


def target_load(E, K, ranks):
    w = ranks.astype(np.float64) ** -S_ZIPF
    p = np.zeros(E)
    free = np.ones(E, dtype=bool)
    budget = float(K)
    while True:  # water-fill: cap at 1, spread the rest by weight
        p[free] = budget * w[free] / w[free].sum()
        over = free & (p > 1.0)
        if not over.any():
            return p
        p[over] = 1.0
        free &= ~over
        budget = K - p[~free].sum()


def main():
    cfg = MI.CONFIGS["v3_decode_fp8"]
    E, K = cfg.E, cfg.K
    gate_w = decode_tensor(MI.gen_gate_w(cfg))
    u = decode_tensor(MI.gen_x(cfg, T=CALIB_T, tid=MI.TID_CALIB_X))
    s = O.affinity(O.router_logits(u, gate_w), "sigmoid")
    perm = MI.permutation(MI.stream_key(cfg.seed, MI.TID_ZIPF_RANK), E).numpy()
    ranks = np.empty(E, dtype=np.int64)
    ranks[perm] = np.arange(1, E + 1)
    p = target_load(E, K, ranks)
    b = np.zeros(E, dtype=np.float32)
    for step in range(300):
        gamma = np.float32(1e-2 if step < 200 else 1e-3)
        idx = O.select_experts(s + b.astype(np.float64)[None, :], cfg.G, cfg.kg, K)[0]
        load = np.bincount(idx.ravel(), minlength=E) / CALIB_T
        b = (b + gamma * np.sign(p - load).astype(np.float32)).astype(np.float32)
    idx = O.select_experts(s + b.astype(np.float64)[None, :], cfg.G, cfg.kg, K)[0]
    load = np.bincount(idx.ravel(), minlength=E) / CALIB_T
    nz = load > 0
    slope = np.polyfit(np.log(ranks[nz]), np.log(load[nz]), 1)[0]
    # experts the 64-token decode batch touches
    u64 = decode_tensor(MI.gen_x(cfg))
    s64 = O.affinity(O.router_logits(u64, gate_w), "sigmoid")
    touched = len(np.unique(O.select_experts(s64 + b.astype(np.float64)[None, :], cfg.G, cfg.kg, K)[0]))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_v3_e256.txt")
    with open(out, "w") as f:
        f.write("# selection bias (float32, hex) of the decode-shaped V3 workload, expert 0..255\n")
        f.write("# written by tests/golden/make_zipf_bias.py (oracle router + the V3 page's +-gamma bias rule)\n")
        f.write(f"# realised popularity slope (log load vs log rank) {slope:.3f}; target -{S_ZIPF}\n")
        f.write(f"# max |load - target| {np.abs(load - p).max():.4f}; experts touched by the 64-token batch {touched}\n")
        for v in b:
            f.write(float(v).hex() + "\n")
    print(f"slope {slope:.3f} touched {touched} max_dev {np.abs(load - p).max():.4f} -> {out}")


if __name__ == "__main__":
    main()
