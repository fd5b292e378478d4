"""Parity checks of GPU results against the oracle.

TEST INFRASTRUCTURE ONLY (used by tests/, __graft_entry__.smoke and the
cpu_baseline leg of bench.py).  Tolerances:

* routing: top-K index sets bit-exact, except tokens whose K-th and (K+1)-th
  oracle logits are closer than 1e-4 (near ties, several answers are correct
  within fp32 rounding); those are counted, and the GPU's choice must still be
  a top-K set within that margin.  Slot order may differ only where the two
  kept logits are within 1e-4 of each other.
* gates: compared per expert id (the dense n-vector G(x)) within 1e-5 absolute;
  for near-tie tokens against the softmax of the GPU's chosen experts.
* output: max|err| <= 2e-2 * RMS and mean|err| <= 2e-3 * RMS, RMS over the
  oracle output, with near-tie tokens evaluated by the oracle on the GPU's
  choice of experts.
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
    order_mismatch: int = 0        # same set, slot order differs beyond a tie
    invalid_choice: int = 0        # near-tie tokens whose choice is not a valid top-K
    gate_max_err: float = 0.0
    forced_idx: np.ndarray | None = field(default=None, repr=False)

    @property
    def ok(self) -> bool:
        return (self.set_mismatch == 0 and self.order_mismatch == 0 and self.invalid_choice == 0
                and self.gate_max_err <= GATE_TOL)


def check_routing(logits: np.ndarray, k: int, idx_gpu: np.ndarray, gate_gpu: np.ndarray,
                  eps: float = TIE_EPS) -> RoutingReport:
    """Compare GPU top-K indices and gates with the oracle's, given oracle logits."""
    T, n = logits.shape
    idx_ref = moe_ref.topk_indices(logits, k)
    tie = moe_ref.near_tie_tokens(logits, k, eps)
    rep = RoutingReport(tokens=T, near_ties=int(tie.sum()))
    idx_gpu = np.asarray(idx_gpu, np.int64)
    forced = idx_ref.copy()
    srt = -np.sort(-logits, axis=1)
    for t in range(T):
        g_set, r_set = set(idx_gpu[t].tolist()), set(idx_ref[t].tolist())
        if tie[t]:
            kth = srt[t, k - 1]
            valid = (len(g_set) == k and all(0 <= e < n for e in g_set)
                     and all(logits[t, e] >= kth - eps for e in g_set))
            if not valid:
                rep.invalid_choice += 1
            forced[t] = idx_gpu[t]
        elif g_set != r_set:
            rep.set_mismatch += 1
        elif not np.array_equal(idx_gpu[t], idx_ref[t]):
            kept = logits[t, idx_gpu[t]]
            if np.any(np.diff(kept) > eps):   # GPU order is not non-increasing within eps
                rep.order_mismatch += 1
    ok_rows = np.all((forced >= 0) & (forced < n), axis=1)
    forced = np.where(ok_rows[:, None], forced, idx_ref)
    g_ref = np.zeros((T, n))
    np.put_along_axis(g_ref, forced, moe_ref.topk_softmax(logits, forced), axis=1)
    g_gpu = np.zeros((T, n))
    safe = np.clip(idx_gpu, 0, n - 1)
    np.put_along_axis(g_gpu, safe, np.asarray(gate_gpu, np.float64), axis=1)
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
    mx, mean, rms = moe_ref.compare_outputs(y_ref, y_gpu)
    return OutputReport(mx, mean, rms)
