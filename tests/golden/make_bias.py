"""Writes the two calibrated router-bias fixtures used by the skewed Nano-shaped layers.

    python tests/golden/make_bias.py

Only the oracle is called (double-precision logits, routing and the aux-loss-free bias step); the
HIP library is not involved. The bias is an *input* of the layer: it is calibrated once, on the
seed-0 tokens and router weights, so that the routing of those tokens has the intended expert
popularity, then frozen as fp32 and stored as hexadecimal floats.

Calibration: 300 aux-loss-free sign steps toward per-expert target loads (aux-loss-free
balancing as named in the Nemotron 3 Nano report summary, section 2.2), step 0.05 decaying by
0.98 per step, starting from zero bias.

  bias_nano_prefill_zipf.txt   T=8192, k=6, E=128: expert of popularity rank r (1-based, rank
      order from a seeded permutation) targets T*k*r^-1.1/sum, water-filled so that no expert
      exceeds T (a token picks an expert at most once) and the total stays T*k.
  bias_nano_fp8_imbalance.txt  T=16384, k=6, E=128: 8 experts fixed at bias -4 (scores lie in
      (0, 1), so they are never picked); the 4 most popular target 10x the mean load (7680);
      the other 116 share the rest equally.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402
from oracle import oracle as O  # noqa: E402

STEPS, GAMMA0, DECAY = 300, 0.05, 0.98


def zipf_targets(T, k, E, s=1.1):
    w = np.arange(1, E + 1, dtype=np.float64) ** -s
    cap = np.zeros(E, bool)
    tgt = np.zeros(E)
    for _ in range(E):
        free = T * k - T * cap.sum()
        tgt = np.where(cap, float(T), free * w / w[~cap].sum())
        over = (tgt > T) & ~cap
        if not over.any():
            break
        cap |= over
    return tgt


def calibrate(cfg, target_by_rank, fixed_by_rank):
    inp = mi.make_layer(cfg, 0, tensors={"x", "W_r"})
    z = O.logits(inp)
    ranks = mi.expert_rank_permutation(0, cfg.E)        # ranks[r] = expert with rank r
    target = np.zeros(cfg.E)
    target[ranks] = target_by_rank
    fixed = np.zeros(cfg.E, bool)
    b = np.zeros(cfg.E)
    for r, v in fixed_by_rank.items():
        fixed[ranks[r]] = True
        b[ranks[r]] = v
    gamma = GAMMA0
    for _ in range(STEPS):
        idx, _, _ = O.route(z, b.astype(np.float32), cfg.k)
        counts = O.dispatch(idx, cfg.E)[0]
        nb = O.bias_update(b, counts, target, gamma)
        b = np.where(fixed, b, nb)
        gamma *= DECAY
    b32 = b.astype(np.float32)
    idx, _, _ = O.route(z, b32, cfg.k)
    counts = O.dispatch(idx, cfg.E)[0]
    return b32, counts[ranks], target_by_rank


def write(fname, b32, header):
    with open(os.path.join(mi.golden_dir(), fname), "w") as f:
        for line in header.strip().splitlines():
            f.write("# " + line + "\n")
        for v in b32:
            f.write(float(v).hex() + "\n")


def main():
    c3 = mi.CONFIGS["nano_prefill_bf16"]
    t3 = zipf_targets(c3.T, c3.k, c3.E)
    b3, n3, _ = calibrate(c3, t3, {})
    write(c3.bias, b3, f"""
Router bias b[E] (fp32, hex) for the Nano-shaped prefill layer, T={c3.T}, E={c3.E}, k={c3.k}.
Zipf(1.1) popularity by rank, water-filled under the per-expert cap T; calibrated on the seed-0
tokens by tests/golden/make_bias.py (oracle only). Realised counts by rank (first 16):
{n3[:16].tolist()}
targets by rank (first 16): {np.round(t3[:16]).astype(int).tolist()}
last 8 by rank: {n3[-8:].tolist()}""")
    print("zipf counts by rank", n3.tolist())

    c5 = mi.CONFIGS["nano_fp8"]
    P = c5.T * c5.k
    t5 = np.zeros(c5.E)
    t5[:4] = 10 * P / c5.E
    t5[4:c5.E - 8] = (P - t5[:4].sum()) / (c5.E - 12)
    b5, n5, _ = calibrate(c5, t5, {r: -4.0 for r in range(c5.E - 8, c5.E)})
    write(c5.bias, b5, f"""
Router bias b[E] (fp32, hex) for the Nano-shaped fp8 layer, T={c5.T}, E={c5.E}, k={c5.k}.
Top 4 experts target 10x the mean load, 8 experts held at -4 (never selected), the rest equal;
calibrated on the seed-0 tokens by tests/golden/make_bias.py (oracle only).
Realised counts by rank: top 4 {n5[:4].tolist()}, last 8 {n5[-8:].tolist()},
others min {n5[4:-8].min()} max {n5[4:-8].max()}, mean load {P / c5.E:.0f}""")
    print("imbalance counts by rank", n5.tolist())


if __name__ == "__main__":
    main()
