"""Writes sigma.json: the draft-noise scale of each stochastic workload,
chosen by bisection so that the mean per-position acceptance probability
sum_y min(p(y), q(y)) over a fixed sample of rows is 0.70.  Here p is the
tempered target softmax and q the noisy draft softmax of the workload's
recipe; this only tunes the input recipe.

Run:  python -m workloads.calibrate_sigma
"""
import json
import os

import numpy as np

from workloads import _boosted_normal_logits, bf16_bits_to_f32, f32_to_bf16_bits

TARGET = 0.70


def _softmax(z):
    z = z.astype(np.float64)
    z -= z.max(axis=-1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=-1, keepdims=True)
    return z


def mean_acceptance(l, noise, sigma, T):
    p = _softmax(l / T)
    q = _softmax(((l + sigma * noise) / T).astype(np.float32)).astype(np.float32).astype(np.float64)
    return float(np.minimum(p, q).sum(axis=-1).mean())


def bisect(l, noise, T):
    lo, hi = 0.0, 4.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if mean_acceptance(l, noise, mid, T) > TARGET:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main():
    rng = np.random.default_rng(20240601)
    V, rows = 128256, 32
    l = _boosted_normal_logits(rng, rows, V).astype(np.float64)
    noise = rng.standard_normal((rows, V))
    s_fp32 = bisect(l, noise, 1.0)
    lb = bf16_bits_to_f32(f32_to_bf16_bits(l.astype(np.float32))).astype(np.float64)
    s_bf16 = bisect(lb, noise, 0.8)
    out = {"chain_fp32": round(s_fp32, 4), "chain_bf16_mixed": round(s_bf16, 4)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sigma.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(out)


if __name__ == "__main__":
    main()
