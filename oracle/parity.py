"""Parity checks of GPU results against the oracle.

TEST INFRASTRUCTURE ONLY (used by tests/, __graft_entry__.smoke and the
cpu_baseline leg of bench.py).  The checks follow the TopK and G(x)
definitions of "Mixtral of Experts", section 2.1: G(x) = Softmax(TopK(x W_g)),
TopK keeping the K largest logits.  Tolerances:

* routing: top-K index sets bit-exact, except tokens whose K-th and (K+1)-th
  oracle logits are closer than 1e-4 (near ties: more than one top-K set is
  correct within fp32 rounding of the logits).  Those are counted, and the
  GPU's choice must still be a top-K set within that margin: K distinct ids,
  every chosen logit at least (K-th largest - 1e-4), and every expert whose
  logit exceeds (K-th largest + 1e-4) chosen.  On every token the slot order
  must be non-increasing in the oracle logits up to 1e-4 (slot 0 holds the
  largest), so two slots may trade places only when their logits are within
  1e-4 of each other.
* gates: compared per expert id (the dense n-vector G(x)) within 1e-5
  absolute; for near-tie tokens against the softmax of the oracle logits of
  the GPU's chosen experts.
* output: max|err| <= 2e-2 * RMS and mean|err| <= 2e-3 * RMS, RMS over the
  oracle output, with near-tie tokens evaluated by the oracle on the GPU's
  choice of experts.

Pinned by tests/test_parity_pins.py against hand-built cases
(tests/golden/parity_checker.json) with faults planted on the "GPU" side.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import moe_ref

TIE_EPS = 1e-4
GATE_TOL = 1e-5
OUT_MAX_TOL = 2e-2
OUT_MEAN_TOL = 2e-3


@dataclass
class RoutingReport:
    tokens: int
    near_ties: int = 0
    set_mismatch: int = 0          # non-tie tokens whose expert set differs
    order_mismatch: int = 0        # slot order not non-increasing within eps
    invalid_choice: int = 0        # near-tie tokens whose choice is not a valid top-K
    gate_max_err: float = 0.0
    forced_idx: np.ndarray | None = field(default=None, repr=False)

    @property
    def ok(self) -> bool:
        return (self.set_mismatch == 0 and self.order_mismatch == 0 and self.invalid_choice == 0
                and self.gate_max_err <= GATE_TOL)


def valid_near_tie_choice(row: np.ndarray, k: int, choice, eps: float = TIE_EPS) -> bool:
    """Whether `choice` (K expert ids) is a top-K set of the logit row `row`
    within eps: K distinct ids in range, none below (K-th largest - eps), and
    none left out above (K-th largest + eps)."""
    n = row.shape[0]
    ids = [int(e) for e in choice]
    if len(set(ids)) != k or any(e < 0 or e >= n for e in ids):
        return False
    kth = -np.sort(-row)[k - 1]
    if any(row[e] < kth - eps for e in ids):
        return False
    must = {e for e in range(n) if row[e] > kth + eps}
    return must <= set(ids)


def check_routing(logits: np.ndarray, k: int, idx_gpu: np.ndarray, gate_gpu: np.ndarray,
                  eps: float = TIE_EPS) -> RoutingReport:
    """Compare GPU top-K indices and gates with the oracle's, given oracle logits."""
    T, n = logits.shape
    idx_ref = moe_ref.topk_indices(logits, k)
    tie = moe_ref.near_tie_tokens(logits, k, eps)
    rep = RoutingReport(tokens=T, near_ties=int(tie.sum()))
    idx_gpu = np.asarray(idx_gpu, np.int64).reshape(T, k)
    forced = idx_ref.copy()
    for t in range(T):
        g = idx_gpu[t]
        in_range = bool(np.all((g >= 0) & (g < n)))
        if tie[t]:
            if not valid_near_tie_choice(logits[t], k, g, eps):
                rep.invalid_choice += 1
                continue
            forced[t] = g
        elif set(g.tolist()) != set(idx_ref[t].tolist()):
            rep.set_mismatch += 1
            continue
        if in_range and np.any(np.diff(logits[t, g]) > eps):
            rep.order_mismatch += 1
    g_ref = np.zeros((T, n))
    np.put_along_axis(g_ref, forced, moe_ref.topk_softmax(logits, forced), axis=1)
    g_gpu = np.zeros((T, n))
    safe = np.clip(idx_gpu, 0, n - 1)
    np.put_along_axis(g_gpu, safe, np.asarray(gate_gpu, np.float64).reshape(T, k), axis=1)
    rep.gate_max_err = float(np.abs(g_ref - g_gpu).max()) if T else 0.0
    rep.forced_idx = forced
    return rep


@dataclass
class OutputReport:
    max_rel: float
    mean_rel: float
    rms: float

    @property
    def ok(self) -> bool:
        return self.max_rel <= OUT_MAX_TOL and self.mean_rel <= OUT_MEAN_TOL


def check_output(y_ref: np.ndarray, y_gpu: np.ndarray) -> OutputReport:
    """Output tolerance: max|err| <= 2e-2 RMS(y_ref), mean|err| <= 2e-3 RMS(y_ref)."""
    y_ref = np.asarray(y_ref, np.float64)
    y_gpu = np.asarray(y_gpu)
    if y_ref.shape != y_gpu.shape:
        raise ValueError(f"shape mismatch: oracle {y_ref.shape}, GPU {y_gpu.shape}")
    if not np.all(np.isfinite(y_gpu)):
        return OutputReport(float("inf"), float("inf"), float(np.sqrt(np.mean(np.square(y_ref)))))
    mx, mean, rms = moe_ref.compare_outputs(y_ref, y_gpu)
    return OutputReport(mx, mean, rms)
