"""Seeded synthetic inputs for the Mixtral-shape sparse MoE layer.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the layer's arithmetic (no routing, no gating, no expert FFN): both
the fp64 oracle under ``oracle/`` and the HIP path consume exactly the arrays
produced here, so the two sides see bit-identical inputs.

Shapes follow Table 1 of "Mixtral of Experts" (dim 4096, hidden_dim 14336,
8 experts, top-2); the paper's Table 1 is reproduced on the garden.houmin.site
translation (section 2) and on the jerryyang.ai blog page.

Recipe (every array is drawn in float32, then rounded to bf16 with
round-to-nearest-even):

* ``x[T][D]``            ~ N(0, 1)
* ``w_gate[D][n]``       ~ N(0, 1/D)
* ``w1[n][D][H]``, ``w3[n][D][H]`` ~ N(0, 1/D)
* ``w2[n][H][D]``        ~ N(0, 1/H)

Seeds: ``SeedSequence(seed).spawn(5)`` gives the x, w_gate, w1, w3, w2 streams
in that order.  The w1/w3/w2 streams are spawned once more per expert, and the
x stream once more per 8192-token chunk, so every block can be drawn on its own
thread and the result does not depend on thread scheduling.

Arrays are returned as ``numpy.uint16`` holding bf16 bit patterns.
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

X_CHUNK = 8192  # tokens per independently seeded block of x

_HERE = os.path.dirname(os.path.abspath(__file__))
SKEW_CALIBRATION_FILE = os.path.join(_HERE, "skew_calibration.json")


# ---------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ---------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even, NaN kept quiet."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = np.isnan(a)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int            # workload number, also the seed offset (seed = 1000 + cfg)
    T: int
    D: int
    H: int
    n: int
    K: int
    weight_seed: int    # Mixtral-shape workloads share one weight set
    skew: bool = False  # add c*u to router columns 0 and 1 (load-imbalance stress)
    chunk: int = 0      # >0: fed to the layer in chunks of this many tokens
    note: str = field(default="", compare=False)

    @property
    def x_seed(self) -> int:
        return 1000 + self.cfg


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 128, 256, 8, 2, 1001,
                     note="T=64 D=128 H=256, drawn in fp32 and rounded to bf16"),
    "decode": Workload("decode", 2, 16, 4096, 14336, 8, 2, 1002,
                       note="Mixtral shape, 16 tokens, memory-bound"),
    "prefill": Workload("prefill", 3, 4096, 4096, 14336, 8, 2, 1002,
                        note="Mixtral shape, 4096 tokens, balanced routing"),
    "skewed": Workload("skewed", 4, 4096, 4096, 14336, 8, 2, 1002, skew=True,
                       note="Mixtral shape, ~60% of token-slots on experts 0 and 1"),
    "large": Workload("large", 5, 32768, 4096, 14336, 8, 2, 1002, chunk=8192,
                      note="Mixtral shape, 32768 tokens streamed as 4 x 8192"),
    # Fine-grained layout: 8 of 160 experts.  The expert width is not given;
    # 768 keeps the layer's expert parameters near Mixtral's (160 * 768 vs
    # 8 * 14336), rounded up to a multiple of 128 columns.
    "fine_prefill": Workload("fine_prefill", 6, 4096, 4096, 768, 160, 8, 1006,
                             note="fine-grained, 8 of 160 experts of width 768, 4096 tokens"),
    "fine_decode": Workload("fine_decode", 7, 16, 4096, 768, 160, 8, 1006,
                            note="fine-grained, 8 of 160 experts of width 768, 16 tokens"),
}


def skew_coefficient() -> float:
    """Calibrated strength c of the skew direction (see oracle/calibrate_skew.py)."""
    with open(SKEW_CALIBRATION_FILE) as f:
        return float(json.load(f)["c"])


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------
def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_bf16(seq: np.random.SeedSequence, shape, scale: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seq))
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return bf16_bits(a)


def _streams(seed: int):
    x_s, g_s, w1_s, w3_s, w2_s = np.random.SeedSequence(seed).spawn(5)
    return x_s, g_s, w1_s, w3_s, w2_s


def make_x(seed: int, T: int, D: int, first_token: int = 0) -> np.ndarray:
    """Tokens [first_token, first_token+T) of the x sequence drawn from ``seed``.

    x is drawn in blocks of ``X_CHUNK`` tokens, block b from its own child seed,
    so any token range can be produced without drawing the tokens before it.
    """
    x_s = _streams(seed)[0]
    if T == 0:
        return np.zeros((0, D), np.uint16)
    b0 = first_token // X_CHUNK
    b1 = (first_token + T - 1) // X_CHUNK
    children = x_s.spawn(b1 + 1)
    parts = []
    for b in range(b0, b1 + 1):
        blk = _normal_bf16(children[b], (X_CHUNK, D), 1.0)
        lo = max(first_token, b * X_CHUNK) - b * X_CHUNK
        hi = min(first_token + T, (b + 1) * X_CHUNK) - b * X_CHUNK
        parts.append(blk[lo:hi])
    return np.ascontiguousarray(np.concatenate(parts, axis=0))


def make_gate_f32(seed: int, D: int, n: int) -> np.ndarray:
    """Router weights w_gate[D][n] in float32, before rounding to bf16."""
    g_s = _streams(seed)[1]
    return np.random.Generator(np.random.PCG64(g_s)).standard_normal(
        (D, n), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))


def make_weights(seed: int, D: int, H: int, n: int):
    """(w_gate_f32[D][n], w1[n][D][H], w3[n][D][H], w2[n][H][D]); the last three
    as bf16 bits, the router weights still in float32."""
    _, g_s, w1_s, w3_s, w2_s = _streams(seed)
    w_gate_f32 = make_gate_f32(seed, D, n)
    w1 = np.empty((n, D, H), np.uint16)
    w3 = np.empty((n, D, H), np.uint16)
    w2 = np.empty((n, H, D), np.uint16)
    jobs = []
    for arr, stream, shape, scale in ((w1, w1_s, (D, H), 1.0 / np.sqrt(D)),
                                      (w3, w3_s, (D, H), 1.0 / np.sqrt(D)),
                                      (w2, w2_s, (H, D), 1.0 / np.sqrt(H))):
        for e, child in enumerate(stream.spawn(n)):
            jobs.append((arr, e, child, shape, scale))

    def run(job):
        arr, e, child, shape, scale = job
        arr[e] = _normal_bf16(child, shape, scale)

    if n * D * H >= (1 << 22):
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return w_gate_f32, w1, w3, w2


def skew_gate(w_gate_f32: np.ndarray, x_bits: np.ndarray, c: float) -> np.ndarray:
    """Add c * u to router columns 0 and 1, u = mean(x) / ||mean(x)||.

    Computed in float64 from the bf16 x values, then the sum is rounded to bf16.
    """
    xm = bf16_to_f32(x_bits).astype(np.float64).mean(axis=0)
    u = xm / np.linalg.norm(xm)
    g = w_gate_f32.astype(np.float64).copy()
    g[:, 0] += c * u
    g[:, 1] += c * u
    return bf16_bits(g.astype(np.float32))


@dataclass
class LayerInputs:
    x: np.ndarray       # uint16 bf16 [T][D]
    w_gate: np.ndarray  # uint16 bf16 [D][n]
    w1: np.ndarray      # uint16 bf16 [n][D][H]
    w3: np.ndarray      # uint16 bf16 [n][D][H]
    w2: np.ndarray      # uint16 bf16 [n][H][D]
    K: int
    skew_c: float = 0.0

    @property
    def shape(self):
        T, D = self.x.shape
        n, _, H = self.w1.shape
        return T, D, H, n, self.K


def make_layer(T: int, D: int, H: int, n: int, K: int, seed: int,
               weight_seed: int | None = None, skew_c: float | None = None,
               x_seed: int | None = None) -> LayerInputs:
    """Inputs of an arbitrary-shape layer (tests use this for ragged sizes)."""
    weight_seed = seed if weight_seed is None else weight_seed
    x_seed = seed if x_seed is None else x_seed
    x = make_x(x_seed, T, D)
    wg_f32, w1, w3, w2 = make_weights(weight_seed, D, H, n)
    if skew_c:
        w_gate = skew_gate(wg_f32, x, skew_c)
    else:
        w_gate = bf16_bits(wg_f32)
        skew_c = 0.0
    return LayerInputs(x, w_gate, w1, w3, w2, K, float(skew_c))


def make_router_inputs(name: str, T: int | None = None):
    """(x, w_gate) of a named workload as bf16 bits, without the expert weights."""
    w = WORKLOADS[name]
    T = w.T if T is None else T
    x = make_x(w.x_seed, T, w.D)
    wg_f32 = make_gate_f32(w.weight_seed, w.D, w.n)
    if w.skew:
        x_full = x if T == w.T else make_x(w.x_seed, w.T, w.D)
        return x, skew_gate(wg_f32, x_full, skew_coefficient())
    return x, bf16_bits(wg_f32)


def make_workload(name: str, T: int | None = None) -> LayerInputs:
    """Inputs of a named workload; ``T`` may cut the token count (prefix of x)."""
    w = WORKLOADS[name]
    T = w.T if T is None else T
    c = skew_coefficient() if w.skew else None
    x = make_x(w.x_seed, T, w.D)
    wg_f32, w1, w3, w2 = make_weights(w.weight_seed, w.D, w.H, w.n)
    if c:
        # the skew direction is measured on the workload's full x
        x_full = x if T == w.T else make_x(w.x_seed, w.T, w.D)
        w_gate = skew_gate(wg_f32, x_full, c)
    else:
        w_gate = bf16_bits(wg_f32)
        c = 0.0
    return LayerInputs(x, w_gate, w1, w3, w2, w.K, float(c))
