"""Calibrate the skew strength c of the load-imbalance workload with the oracle.

Test infrastructure only.  The load-imbalance workload adds c * u to router
columns 0 and 1 (u = mean(x)/||mean(x)||) so that about 60% of the token-slots
land on experts 0 and 1.  With the literal strength 0.05 only ~27% do, so c is
found here by bisection on the seeded inputs, using only the oracle's router
and top-K, and written to ``moe_synth/skew_calibration.json``.

Run:  python -m oracle.calibrate_skew
"""
from __future__ import annotations

import json
import sys

import numpy as np

import moe_synth
from oracle import moe_ref

TARGET = 0.60


def share_on_01(x_bits, wg_f32, c: float, k: int) -> tuple[float, np.ndarray]:
    wg = moe_synth.skew_gate(wg_f32, x_bits, c)
    idx = moe_ref.topk_indices(moe_ref.router_logits(x_bits, wg), k)
    counts = np.bincount(idx.ravel(), minlength=wg_f32.shape[1])
    return float(counts[:2].sum() / idx.size), counts


def calibrate(name: str = "skewed", tol: float = 0.002):
    w = moe_synth.WORKLOADS[name]
    x = moe_synth.make_x(w.x_seed, w.T, w.D)
    wg_f32 = moe_synth.make_gate_f32(w.weight_seed, w.D, w.n)
    lo, hi = 0.0, 4.0
    c, s, counts = hi, None, None
    for _ in range(60):
        c = 0.5 * (lo + hi)
        s, counts = share_on_01(x, wg_f32, c, w.K)
        if abs(s - TARGET) <= tol:
            break
        if s < TARGET:
            lo = c
        else:
            hi = c
    literal, _ = share_on_01(x, wg_f32, 0.05, w.K)
    return dict(workload=name, c=round(c, 6), share_01=s, counts=[int(v) for v in counts],
                target=TARGET, literal_c=0.05, literal_share_01=literal)


if __name__ == "__main__":
    res = calibrate()
    # make sure the stored constant reproduces the stored share
    print(json.dumps(res))
    with open(moe_synth.SKEW_CALIBRATION_FILE, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    sys.exit(0)
