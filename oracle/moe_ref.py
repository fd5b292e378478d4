"""Oracle: the Mixtral sparse MoE layer written out plainly, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, as the reference the HIP kernels
are checked against.  It shares no code with the HIP path; both sides only
share the seeded input generator ``moe_synth``.

What it computes (sources are the pages on Mixtral of Experts):

* MoE output  y = sum_i G(x)_i * E_i(x)
  -- "Mixtral of Experts", section 2.1 (Sparse Mixture of Experts), first
  display equation (garden.houmin.site translation).
* Gate  G(x) = Softmax(TopK(x . W_g)), TopK keeps the K largest logits and sets
  the rest to -inf -- same section, the G(x) and TopK definitions; the same
  statement in prose is on the jerryyang.ai blog page (gating paragraph).
* Experts are SwiGLU blocks, K = 2, and y = sum_i Softmax(Top2(x W_g))_i *
  SwiGLU_i(x) -- same section, last display equation.

Readings where the pages are silent:

* SwiGLU_i(x) = (silu(x w1_i) * (x w3_i)) w2_i, silu(z) = z / (1 + e^-z),
  no biases; row-vector convention x . W, with W_g[D][n], w1/w3[D][H], w2[H][D].
* Ties in TopK go to the lower expert index; slot 0 holds the larger logit.
* exp(-inf) = 0 exactly, so the softmax runs over the K kept logits only,
  after subtracting the largest; K = 1 gives a gate of exactly 1.
* The weighted sum over the K chosen experts is taken in slot order.
* Inputs are the bf16 values the GPU consumes, widened exactly to float64;
  nothing inside the oracle is rounded.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against something other than itself (hand-worked values under
``tests/golden/``, a dense evaluation of all experts, the K = n dense softmax
mixture, brute force over expert subsets, identical-expert collapse to one
FFN, permutation invariance, and the routing closed forms of Table 5).
"""
from __future__ import annotations

import itertools

import numpy as np


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------
def from_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return from_bf16(a)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# router and gate  (section 2.1: G(x) := Softmax(TopK(x . W_g)))
# ---------------------------------------------------------------------------
def router_logits(x, w_gate) -> np.ndarray:
    """l = x . W_g, the "linear layer" whose Top-K logits feed the softmax."""
    return as_f64(x) @ as_f64(w_gate)


def topk_indices(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the K largest logits per row, ordered by (-l_i, i).

    A stable sort of -l keeps equal logits in index order, so the lower expert
    index wins a tie and slot 0 holds the largest logit.
    """
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_softmax(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over TopK(l): entries outside the top-K are -inf and get exactly 0,
    so only the K kept logits enter the normalisation.  Returned per slot."""
    kept = np.take_along_axis(logits, idx, axis=1)
    m = kept.max(axis=1, keepdims=True)
    e = np.exp(kept - m)
    return e / e.sum(axis=1, keepdims=True)


def dense_gate(logits: np.ndarray, k: int, idx: np.ndarray | None = None) -> np.ndarray:
    """G(x) as the full n-vector (zeros outside the chosen experts)."""
    if idx is None:
        idx = topk_indices(logits, k)
    g = np.zeros_like(logits)
    np.put_along_axis(g, idx, topk_softmax(logits, idx), axis=1)
    return g


def near_tie_tokens(logits: np.ndarray, k: int, eps: float = 1e-4) -> np.ndarray:
    """Tokens whose K-th and (K+1)-th largest logits differ by less than eps.

    For these, more than one top-K set is correct within fp32 rounding."""
    n = logits.shape[1]
    if k >= n:
        return np.zeros(logits.shape[0], dtype=bool)
    s = -np.sort(-logits, axis=1)
    return (s[:, k - 1] - s[:, k]) < eps


# ---------------------------------------------------------------------------
# expert (section 2.1: SwiGLU experts)
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(xr: np.ndarray, w1e, w3e, w2e) -> np.ndarray:
    """E(x) = (silu(x w1) * (x w3)) w2 for a block of rows."""
    a = xr @ as_f64(w1e)
    b = xr @ as_f64(w3e)
    return (silu(a) * b) @ as_f64(w2e)


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
def moe_layer(x, w_gate, w1, w3, w2, k: int, forced_idx=None, return_slots=False):
    """Sparse evaluation: y_t = sum over slots s of g_{t,s} * E_{i_{t,s}}(x_t).

    Only the experts a token is routed to are evaluated (skipping zero-gate
    experts is exact, section 2.1).  ``forced_idx`` overrides the top-K choice
    (gates are then the softmax over the forced experts' logits), which is how
    near-tie tokens are compared with a GPU that picked the other candidate.

    Returns dict(y[T][D], idx[T][K], gate[T][K], logits[T][n]).
    """
    xf = as_f64(x)
    T, D = xf.shape
    n = np.asarray(w1).shape[0]
    logits = router_logits(xf, w_gate)
    idx = topk_indices(logits, k) if forced_idx is None else np.asarray(forced_idx, np.int64)
    gate = topk_softmax(logits, idx)
    E = np.zeros((T, k, D))  # expert output per (token, slot)
    for e in range(n):
        tok, slot = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        E[tok, slot] = swiglu_expert(xf[tok], w1[e], w3[e], w2[e])
    y = np.zeros((T, D))
    for s in range(k):  # slot order
        y += gate[:, s:s + 1] * E[:, s]
    out = dict(y=y, idx=idx, gate=gate, logits=logits)
    if return_slots:
        out["E"] = E
    return out


def moe_layer_rows(x_rows, w_gate, w1, w3, w2, k: int, forced_idx=None):
    """The layer on a subset of tokens (each token is independent, section 2.1:
    the MoE layer is applied to every token separately).  Used for sampled
    parity at full size."""
    return moe_layer(x_rows, w_gate, w1, w3, w2, k, forced_idx=forced_idx)


def moe_layer_dense(x, w_gate, w1, w3, w2, k: int) -> np.ndarray:
    """Dense evaluation: every expert on every token, masked by the n-vector G(x).

    Equal to ``moe_layer`` because experts with a zero gate contribute nothing."""
    xf = as_f64(x)
    g = dense_gate(router_logits(xf, w_gate), k)
    n = np.asarray(w1).shape[0]
    y = np.zeros((xf.shape[0], np.asarray(w2).shape[2]))
    for e in range(n):
        y += g[:, e:e + 1] * swiglu_expert(xf, w1[e], w3[e], w2[e])
    return y


def moe_layer_bruteforce(x, w_gate, w1, w3, w2, k: int) -> np.ndarray:
    """Tiny inputs only: enumerate every K-subset of experts, keep the one with
    the largest summed logit (first in lexicographic order on a tie, which is
    the lowest-index rule), and evaluate everything with scalar Python loops."""
    xf, wg = as_f64(x), as_f64(w_gate)
    W1, W3, W2 = as_f64(w1), as_f64(w3), as_f64(w2)
    T, D = xf.shape
    n, _, H = W1.shape
    y = np.zeros((T, W2.shape[2]))
    for t in range(T):
        l = [sum(xf[t, d] * wg[d, i] for d in range(D)) for i in range(n)]
        best, best_sum = None, -np.inf
        for sub in itertools.combinations(range(n), k):
            s = sum(l[i] for i in sub)
            if s > best_sum:
                best, best_sum = sub, s
        m = max(l[i] for i in best)
        w = {i: np.exp(l[i] - m) for i in best}
        z = sum(w.values())
        for i in best:
            g = w[i] / z
            for o in range(W2.shape[2]):
                acc = 0.0
                for j in range(H):
                    a = sum(xf[t, d] * W1[i, d, j] for d in range(D))
                    b = sum(xf[t, d] * W3[i, d, j] for d in range(D))
                    acc += (a / (1.0 + np.exp(-a))) * b * W2[i, j, o]
                y[t, o] += g * acc
    return y


# ---------------------------------------------------------------------------
# routing statistics (section 5: Figure 7 shares, Table 5 repetition rates)
# ---------------------------------------------------------------------------
def expert_share(idx: np.ndarray, n: int) -> np.ndarray:
    """Fraction of token-slots (first or second choice) assigned to each expert."""
    return np.bincount(idx.ravel(), minlength=n) / idx.size


def consecutive_repeat(idx: np.ndarray):
    """(first-choice repeat rate, either-choice repeat rate) between tokens t, t+1.

    first: token t and t+1 have the same first-choice expert.
    either: some expert appears among the chosen experts of both tokens."""
    a, b = idx[:-1], idx[1:]
    first = np.mean(a[:, 0] == b[:, 0])
    either = np.mean((a[:, :, None] == b[:, None, :]).any(axis=(1, 2)))
    return float(first), float(either)


def route_stats(idx: np.ndarray, n: int) -> dict:
    """Exact routing counts over a [T][K] choice array ("Mixtral of Experts",
    section 5: the per-expert shares of Figure 7 / Figure 9 as first choice and
    as either choice, and the consecutive-token repetitions of Table 5).

    Ids outside [0, n) are not counted and match nothing.  Returns plain ints:
    first[e], any[e] (slot counts), repeat_first (tokens t < T-1 whose first
    choice equals token t+1's) and repeat_either (tokens t < T-1 sharing any
    chosen expert with token t+1)."""
    idx = np.asarray(idx)
    T = idx.shape[0]
    first = [0] * n
    anyc = [0] * n
    rep_first = rep_either = 0
    for t in range(T):
        row = [int(v) for v in idx[t]]
        if 0 <= row[0] < n:
            first[row[0]] += 1
        for v in row:
            if 0 <= v < n:
                anyc[v] += 1
        if t + 1 < T:
            nxt = [int(v) for v in idx[t + 1]]
            valid = [v for v in row if 0 <= v < n]
            if 0 <= row[0] < n and nxt[0] == row[0]:
                rep_first += 1
            if any(v in nxt for v in valid):
                rep_either += 1
    return {"first": first, "any": anyc, "repeat_first": rep_first, "repeat_either": rep_either}


# ---------------------------------------------------------------------------
# parity comparison helper used by the tests
# ---------------------------------------------------------------------------
def compare_outputs(y_ref: np.ndarray, y_test: np.ndarray):
    """(max|err|/RMS, mean|err|/RMS, RMS) with RMS over all entries of y_ref."""
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    err = np.abs(np.asarray(y_test, np.float64) - y_ref)
    if rms == 0.0:
        return float(err.max(initial=0.0)), float(err.mean() if err.size else 0.0), rms
    return float(err.max(initial=0.0) / rms), float((err.mean() if err.size else 0.0) / rms), rms
