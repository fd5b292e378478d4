"""Benchmark of the Mixtral sparse MoE layer (libmoe) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole layer (router, permute, both expert products,
combine) over one batch of synthetic Mixtral-shape input already resident in
HBM.  Workloads (seeded, see moe_synth): prefill (T=4096, the default), decode
(T=16), skewed (T=4096, ~60% of token-slots on two experts), large (T=32768
fed as 4 chunks of 8192 through one workspace), tiny, and the fine-grained
layout fine_prefill / fine_decode (8 of 160 experts of width 768, T=4096 / 16).

Prints one JSON line: the headline workload (--workload, prefill by default)
at the top level and, unless --no-side, one sub-record per other workload
under "workloads" (decode, skewed, large, tiny, fine_prefill, fine_decode;
fewer steps each), each with its time, throughput, stage breakdown and the
dominant kernel's roofline.  Every 4th timed step records HIP events on the
layer's stream around the dominant kernel (the first expert product: x.w1,
x.w3 + silu), whose event-timed average launch the roofline object uses; the
per-stage breakdown comes from a separate pass with every stage boundary
recorded (each recorded event costs the stream a few microseconds).
The cpu_baseline object times the fp64 oracle on a bounded sample of the same
workload on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_synth  # noqa: E402

METRIC = "MoE-layer tokens/sec + TFLOP/s (% MFMA peak), Mixtral shape, top-2 of 8, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)


# ---------------------------------------------------------------------------
# algorithmic work (what the method must do; padding and skipped experts excluded)
# ---------------------------------------------------------------------------
def layer_flops(T, D, H, n, K):
    """2*T*K*3*D*H expert multiply-adds x2 plus the router's 2*T*D*n."""
    return 2 * T * K * 3 * D * H + 2 * T * D * n


def up_flops(T, D, H, K):
    return 2 * 2 * T * K * D * H


def up_weight_bytes(touched, D, H):
    return touched * 2 * D * H * 2


def mixtral_params(dim=4096, n_layers=32, head_dim=128, hidden=14336, n_heads=32,
                   n_kv_heads=8, vocab=32000, n_experts=8, top_k=2):
    """(total, active) parameters of the whole model from Table 1 shapes; used to
    check the FLOP/byte accounting against the pages' 46.7B / 13B."""
    attn = dim * n_heads * head_dim * 2 + dim * n_kv_heads * head_dim * 2
    expert = 3 * dim * hidden
    router = dim * n_experts
    norms = 2 * dim
    per_layer_total = attn + n_experts * expert + router + norms
    per_layer_active = attn + top_k * expert + router + norms
    emb = 2 * vocab * dim + dim
    return n_layers * per_layer_total + emb, n_layers * per_layer_active + emb


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (timing on the layer's own stream)
# ---------------------------------------------------------------------------
class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, count):
        out = []
        for _ in range(count):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        self.made += out
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(ev))
        self.made = []


STAGES = ("route", "permute", "up", "down", "combine")
# the dominant kernel's launches are event-timed on every EVENT_EVERY-th timed step
EVENT_EVERY = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def cpu_baseline(name, inputs, sample_tokens, min_seconds=10.0):
    """Time the fp64 oracle (as it stands) on the first `sample_tokens` tokens,
    repeated until at least `min_seconds` of wall time have passed."""
    from threadpoolctl import threadpool_info
    from oracle import moe_ref
    L = inputs
    reps = 0
    t0 = time.perf_counter()
    while True:
        moe_ref.moe_layer(L.x[:sample_tokens], L.w_gate, L.w1, L.w3, L.w2, L.K)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = max(threads) if threads else 1
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": reps * sample_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the {name} workload with its full weights, "
                      f"fp64 numpy oracle run {reps}x, {dt:.1f} s wall", "cpu": cpu}


def crossover(args, torch, moe):
    """Small-batch sweep ("Mixtral of Experts", section 3, remark on small
    batches; the summary's limitations): at each T the layer runs once with the
    weight-streaming expert path (while T <= decode_max_tokens) and once with
    the tiled matrix-core path, same inputs and weights (the Mixtral-shape
    decode weight set).  Reports per-step GPU time, the weight bytes of the
    touched experts per second, TFLOP/s, and the largest T at which streaming
    is faster."""
    w = moe_synth.WORKLOADS["decode"]
    D, H, n, K = w.D, w.H, w.n, w.K
    log("[crossover] generating Mixtral-shape weights")
    L = moe_synth.make_workload("decode")
    wg, w1, w3, w2 = (to_dev(a) for a in (L.w_gate, L.w1, L.w3, L.w2))
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    rows = []
    for T in (1, 2, 4, 8, 16, 24, 32, 48, 64, 80, 96, 112, 128, 192, 256):
        x = to_dev(moe_synth.make_x(w.x_seed, T, D))
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
        out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
        row = {"T": T}
        for name, path in (("stream", moe.PATH_STREAM), ("tiled", moe.PATH_TILED)):
            nbytes = moe.workspace_bytes(moe.problem(T, D, H, n, K, path=path))
            if nbytes == 0:  # streaming beyond the batch sizes it supports
                continue
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
            run = lambda e=None: moe.forward(x, wg, w1, w3, w2, K, out=out, topk_idx=idx,
                                             workspace=ws, stream=stream, events=e, path=path)
            for _ in range(args.warmup):
                run()
            # only the first and last events: each recorded event costs the
            # stream a few microseconds
            evs = [ev.create(2) for _ in range(args.steps)]
            for e2 in evs:
                run([e2[0], None, None, None, None, e2[1]])
            torch.cuda.synchronize()
            ms = float(np.median([ev.elapsed_ms(e2[0], e2[1]) for e2 in evs]))
            touched = int((np.bincount(idx.cpu().numpy().ravel(), minlength=n) > 0).sum())
            wbytes = touched * 3 * D * H * 2
            row[name] = {"ms": ms, "weight_gbs": wbytes / (ms / 1e3) / 1e9,
                         "tflops": layer_flops(T, D, H, n, K) / (ms / 1e3) / 1e12}
            log(f"[crossover] T={T} {name}: {ms * 1e3:.1f} us")
        rows.append(row)
    ev.close()
    faster = [r["T"] for r in rows if "stream" in r and r["stream"]["ms"] < r["tiled"]["ms"]]
    rec = {"metric": "small-batch crossover: layer time by expert-product path",
           "unit": "ms", "data": "synthetic", "dtype": "bf16",
           "config": {"workload": "decode weights, T swept", "dim": D, "hidden": H, "n_experts": n,
                      "top_k": K, "steps": args.steps, "warmup": args.warmup},
           "rows": rows, "stream_faster_up_to_T": max(faster) if faster else 0,
           "library_threshold_T": moe.decode_max_tokens()}
    print(json.dumps(rec), flush=True)
    return 0


def weight_data(args, torch, moe):
    """The layer at a workload's shape with the same x and router but four
    kinds of expert weights: the random weights it is benchmarked with, all
    zero, one constant (2^-7) and random signs of that constant.  Every run does
    the same work in the same order; only the values the matrix cores multiply
    differ.  Under the board's power limit the clock follows the switching
    activity of that data, so the differences in time are the share of the
    expert products' cost that power, not the kernels' structure, decides."""
    name = args.workload
    w = moe_synth.WORKLOADS[name]
    order = args.weight_data.split(",")
    unknown = [k for k in order if k not in ("random", "zero", "const", "sign")]
    if unknown:
        raise SystemExit(f"--weight-data: unknown kinds {unknown}; known: random, zero, const, sign")
    log(f"[weight-data] generating {name} inputs")
    L = moe_synth.make_workload(name)
    x, wg = to_dev(L.x), to_dev(L.w_gate)
    rand = tuple(to_dev(a) for a in (L.w1, L.w3, L.w2))
    const = 2.0 ** -7
    kinds = {
        "random": lambda: rand,
        "zero": lambda: tuple(torch.zeros_like(t) for t in rand),
        "const": lambda: tuple(torch.full_like(t, const) for t in rand),
        "sign": lambda: tuple((torch.sign(t.float()) * const).to(torch.bfloat16) for t in rand),
    }
    from sparse_moe_layer_gemv_amd.profiling import load_traffic
    rows = []
    for kind in order:
        w1, w3, w2 = kinds[kind]()
        r = time_workload(name, L, (x, wg, w1, w3, w2), args.steps, args.warmup, torch, moe,
                          load_traffic, HipEvents())
        rows.append({"weights": kind, "ms_per_step": r["ms_per_step"],
                     "step_gpu_ms": r["step_gpu_ms"]["median"],
                     "mfma_peak_frac": r.get("mfma_peak_frac"),
                     "stage_us": {k: round(v * 1e3, 1) for k, v in r["stage_ms"].items()}})
        log(f"[weight-data] {kind}: {r['ms_per_step']:.4f} ms/step")
        del w1, w3, w2
    rec = {"metric": "layer time by expert-weight data (same routing and work)", "unit": "ms",
           "data": "synthetic", "dtype": "bf16",
           "config": {"workload": name, "tokens": w.T, "dim": w.D, "hidden": w.H,
                      "n_experts": w.n, "top_k": w.K, "steps": args.steps,
                      "warmup": args.warmup},
           "rows": rows}
    print(json.dumps(rec), flush=True)
    return 0


ROTATION_BYTES = 1 << 30  # inputs rotated per stage, so that every call reads from HBM


def stages_alone(args, torch, moe):
    """Router, permute and combine, each timed alone at a workload's shape.

    The stage's large inputs are cycled through copies totalling at least
    1 GiB (x for the router, the fp32 expert rows for the combine), far beyond
    the 4 MiB L2 per XCD and the 256 MiB MALL, so the bytes a call reads come
    from HBM.  Bytes per call are the algorithmic ones:
      router:  T*D*2 (x) + D*n*2 (W_g) + T*K*8 (topk_idx, topk_gate)
      permute: T*K*4 read; n*4 + (n+1)*4 + cap*4 + T*K*4 written
      combine: T*K*D*4 (the token-slots' expert rows) + T*K*8 + T*D*4 (out)
    Time per call is the hipEvent time of `steps` back-to-back calls on the
    current stream, divided by `steps`.  Prints one JSON line."""
    w = moe_synth.WORKLOADS[args.workload]
    T, D, n, K = w.T, w.D, w.n, w.K
    log(f"[stages] {args.workload}: T={T} D={D} n={n} K={K}")
    xh, wgh = moe_synth.make_router_inputs(args.workload)
    x0, wg = to_dev(xh), to_dev(wgh)
    p = moe.problem(T, D, 8, n, K)
    cap = moe.capacity_rows(p)
    rws = torch.empty(max(moe.route_workspace_bytes(p), 256), dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")

    def timed(fn, nbuf):
        for i in range(min(args.warmup, nbuf) + 1):
            fn(i % nbuf)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i % nbuf)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps * 1e3  # us per call

    res = {}
    # router over rotating copies of x
    nx = max(1, -(-ROTATION_BYTES // (T * D * 2)))
    xs = [x0.clone() for _ in range(nx)]
    us = timed(lambda i: moe.route(xs[i], wg, K, topk_idx=idx, topk_gate=gate, workspace=rws), nx)
    res["route"] = {"us": us, "bytes": T * D * 2 + D * n * 2 + T * K * 8, "rotated_bytes": nx * T * D * 2}
    del xs
    # permute: a few kilobytes in and out, so latency-bound; rotated copies of
    # the routing all the same
    ni = 64
    idxs = [idx.clone() for _ in range(ni)]
    outs = {"expert_count": torch.empty(n, dtype=torch.int32, device="cuda:0"),
            "expert_offset": torch.empty(n + 1, dtype=torch.int32, device="cuda:0"),
            "row_slot": torch.empty(cap, dtype=torch.int32, device="cuda:0"),
            "slot_row": torch.empty(T * K, dtype=torch.int32, device="cuda:0")}
    us = timed(lambda i: moe.permute(idxs[i], n, out=outs), ni)
    res["permute"] = {"us": us, "bytes": T * K * 4 + (2 * n + 1) * 4 + cap * 4 + T * K * 4}
    perm = moe.permute(idx, n)
    # combine over rotating expert-row buffers (one fp32 partial, as moe_combine takes)
    ny = max(1, -(-ROTATION_BYTES // (cap * D * 4)))
    ys = [torch.empty((cap, D), dtype=torch.float32, device="cuda:0").uniform_(-1, 1)
          for _ in range(ny)]
    out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
    us = timed(lambda i: moe.combine(ys[i], perm["slot_row"], gate, out=out), ny)
    res["combine"] = {"us": us, "bytes": T * K * D * 4 + T * K * 8 + T * D * 4,
                      "rotated_bytes": ny * cap * D * 4}
    del ys
    for r in res.values():
        r["gbs"] = r["bytes"] / (r["us"] * 1e-6) / 1e9
        r["hbm_frac"] = r["gbs"] / PEAK_HBM_GBS
    rec = {"metric": "stage-alone time and HBM throughput (router, permute, combine)",
           "unit": "GB/s", "data": "synthetic", "dtype": "bf16 in, fp32 out",
           "config": {"workload": args.workload, "tokens": T, "dim": D, "n_experts": n,
                      "top_k": K, "steps": args.steps},
           "peak_hbm_gbs": PEAK_HBM_GBS, "stages": res}
    print(json.dumps(rec), flush=True)
    return 0


def time_workload(name, L, dev, steps, warmup, torch, moe, load_traffic, ev, tokens=None):
    """Time `steps` layer passes of workload `name` (after `warmup` untimed
    ones) on inputs already in HBM.  dev: the uploaded x, w_gate, w1, w3, w2.
    Returns the per-workload record (time, throughput, stage breakdown and
    the dominant kernel's roofline)."""
    w = moe_synth.WORKLOADS[name]
    T, D, H, n, K = (tokens or w.T), w.D, w.H, w.n, w.K
    chunk = min(w.chunk or T, T)
    x, wg, w1, w3, w2 = dev
    out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(moe.workspace_bytes(moe.problem(chunk, D, H, n, K)), dtype=torch.uint8,
                     device="cuda:0")
    stream = torch.cuda.current_stream()
    n_chunks = (T + chunk - 1) // chunk

    def step(events_for_step=None):
        for c in range(n_chunks):
            c0, c1 = c * chunk, min(T, (c + 1) * chunk)
            e6 = None if events_for_step is None else events_for_step[c]
            moe.forward(x[c0:c1], wg, w1, w3, w2, K, out=out[c0:c1], topk_idx=idx[c0:c1],
                        topk_gate=gate[c0:c1], workspace=ws, stream=stream, events=e6)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {name}: warmup done ({warmup} steps); timing {steps} steps")

    # Every recorded event costs the stream a few microseconds, so the timed
    # steps record only the two events around the first expert product (the
    # dominant kernel, whose launches the roofline needs timed live), and only
    # on every EVENT_EVERY-th step; the other stage boundaries are taken in a
    # separate pass afterwards.
    sampled = list(range(0, steps, EVENT_EVERY))
    up_evs = {s: [ev.create(2) for _ in range(n_chunks)] for s in sampled}
    timed = [[[None, None, e2[0], e2[1], None, None] for e2 in up_evs[s]] if s in up_evs else None
             for s in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(steps):
        step(timed[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"[bench] {name}: timed region done: {wall * 1e3:.2f} ms")
    up_timed = [ev.elapsed_ms(e2[0], e2[1]) for s in sampled for e2 in up_evs[s]]

    # stage breakdown: all six events, in a pass of its own
    prof_steps = max(1, min(steps, 10))
    evs = [[ev.create(6) for _ in range(n_chunks)] for _ in range(prof_steps)]
    for s in range(prof_steps):
        step(evs[s])
    torch.cuda.synchronize()
    stage_ms = {k: [] for k in STAGES}
    for s in range(prof_steps):
        for c in range(n_chunks):
            e6 = evs[s][c]
            for i, k in enumerate(STAGES):
                stage_ms[k].append(ev.elapsed_ms(e6[i], e6[i + 1]))
    # per-step layer time on the GPU with every stage event recorded (first
    # stage start to last stage end)
    step_gpu_ms = [ev.elapsed_ms(evs[s][0][0], evs[s][n_chunks - 1][len(STAGES)])
                   for s in range(prof_steps)]
    ev.close()
    # per-launch averages (one launch of each stage per chunk); the first
    # expert product's from the timed steps
    stage_avg = {k: float(np.mean(v)) for k, v in stage_ms.items()}
    up_avg_timed = float(np.mean(up_timed))

    ms_per_step = wall * 1e3 / steps
    flops = layer_flops(T, D, H, n, K)
    tflops = flops / (ms_per_step / 1e3) / 1e12

    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=n)
    touched = int((counts > 0).sum())
    decode = chunk <= moe.decode_max_tokens()
    kernel = "decode_up" if decode else "grouped_up"
    # HBM bytes per launch from the stored counter runs of this exact kernel
    # source (None once the source has changed since they were taken)
    tr = load_traffic(kernel, name) if tokens in (None, w.T) else None
    traffic = None if tr is None else tr["bytes_per_launch"]
    # The dominant kernel's bound: the larger of its time at the matrix-core
    # peak (algorithmic FLOPs) and at the HBM peak (algorithmic bytes: w1 and
    # w3 of every touched expert once, plus x read and h written once by the
    # tiled kernel).  The weight-streaming kernel is bound by the weights.
    w_bytes = up_weight_bytes(touched, D, H)
    if decode:
        per_launch_bytes = w_bytes
        per_launch_flops = 0
    else:
        per_launch_bytes = w_bytes + chunk * D * 2 + chunk * K * H * 2
        per_launch_flops = up_flops(chunk, D, H, K)
    up_s = up_avg_timed / 1e3
    if per_launch_flops / (PEAK_BF16_TFLOPS * 1e12) >= per_launch_bytes / (PEAK_HBM_GBS * 1e9):
        achieved = per_launch_flops / up_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": kernel,
                "algorithmic_per_launch": per_launch_flops, "traffic_unit": "HBM bytes per launch"}
    else:
        achieved = per_launch_bytes / up_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": kernel,
                "algorithmic_per_launch": per_launch_bytes, "traffic_unit": "HBM bytes per launch"}
    if per_launch_flops:
        roof["tflops"] = per_launch_flops / up_s / 1e12
    roof["kernel_ms"] = up_avg_timed  # event-timed average launch over the sampled timed steps
    roof["kernel_launches_timed"] = len(up_timed)

    rec = {
        "workload": name, "tokens": T, "dim": D, "hidden": H, "n_experts": n, "top_k": K,
        "chunk": chunk, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step,
        "tokens_per_s": T / (ms_per_step / 1e3),
        "tflops": tflops,
        "mfma_peak_frac": tflops / PEAK_BF16_TFLOPS,
        # per-stage breakdown and event-timed layer time from the separate pass
        # with all six stage events recorded
        "stage_ms": stage_avg,
        "step_gpu_ms": {"median": float(np.median(step_gpu_ms)), "min": float(np.min(step_gpu_ms)),
                        "mean": float(np.mean(step_gpu_ms))},
        "stage_pass_steps": prof_steps,
        "expert_counts": counts.tolist(),
        "roofline": roof,
    }
    if decode:
        # the whole layer against HBM: every touched expert's three matrices
        # once, plus x, W_g, out and the routing
        total_bytes = touched * 3 * D * H * 2 + T * D * 2 + D * n * 2 + T * D * 4 + T * K * 8
        rec["hbm_gbs_layer"] = total_bytes / (ms_per_step / 1e3) / 1e9
        rec["hbm_peak_frac_layer"] = rec["hbm_gbs_layer"] / PEAK_HBM_GBS
    return rec


# Workloads timed beside the headline one in the default run, with the steps
# each gets (a step of `large` is 4 layer calls of 8192 tokens).
SIDE_WORKLOADS = (("decode", 50), ("skewed", 30), ("large", 10), ("tiny", 50),
                  ("fine_prefill", 30), ("fine_decode", 50))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=sorted(moe_synth.WORKLOADS))
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the headline workload with this many tokens (a prefix of its x)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="time only the headline workload (no per-workload sub-records)")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens for the oracle timing (default: a bounded sample per workload)")
    ap.add_argument("--crossover", action="store_true",
                    help="small-batch sweep: time both expert-product paths for T = 1..256 and "
                         "print one JSON line with the measured crossover")
    ap.add_argument("--weight-data", nargs="?", const="random,zero,const,sign,random,zero",
                    metavar="KINDS",
                    help="time the workload with random, zero, constant and random-sign expert "
                         "weights, in the comma-separated order KINDS (same routing and work; "
                         "one JSON line)")
    ap.add_argument("--stages", action="store_true",
                    help="router, permute and combine each timed alone at the workload's shape, "
                         "over rotating inputs of at least 1 GiB (one JSON line)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "libmoe is a single-GPU build: each GPU runs the whole layer "
                                   "on its own share of tokens and there is no cross-GPU step; "
                                   "run with --gpus 1"}))
        return 2

    import torch
    import sparse_moe_layer_gemv_amd as moe
    from sparse_moe_layer_gemv_amd.profiling import load_traffic

    if args.crossover:
        return crossover(args, torch, moe)
    if args.stages:
        return stages_alone(args, torch, moe)
    if args.weight_data:
        return weight_data(args, torch, moe)

    names = [args.workload]
    side = {}
    if not args.no_side:
        side = {nm: min(st, args.steps) for nm, st in SIDE_WORKLOADS if nm != args.workload}
        names += list(side)
    # one upload per weight set: the Mixtral-shape workloads share theirs
    uploaded = {}
    records = {}
    head_inputs = None
    for name in names:
        w = moe_synth.WORKLOADS[name]
        log(f"[bench] generating {name} inputs T={w.T} D={w.D} H={w.H} n={w.n} K={w.K}")
        t0 = time.perf_counter()
        tok = args.tokens if (name == args.workload and args.tokens) else None
        L = moe_synth.make_workload(name, T=tok)
        log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
        key = (w.weight_seed, w.D, w.H, w.n)
        if key not in uploaded:
            uploaded.clear()  # the previous weight set is no longer needed
            torch.cuda.empty_cache()
            uploaded[key] = tuple(to_dev(a) for a in (L.w1, L.w3, L.w2))
        dev = (to_dev(L.x), to_dev(L.w_gate)) + uploaded[key]
        steps = args.steps if name == args.workload else side[name]
        warmup = args.warmup if name == args.workload else min(args.warmup, 3)
        records[name] = time_workload(name, L, dev, steps, warmup, torch, moe, load_traffic,
                                      HipEvents(), tokens=tok)
        del dev
        if name == args.workload:
            head_inputs = L
        else:
            del L

    h = records[args.workload]
    rec = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": h["tokens"], "dim": h["dim"],
                   "hidden": h["hidden"], "n_experts": h["n_experts"], "top_k": h["top_k"],
                   "chunk": h["chunk"], "parallelism": "none"},
    }
    for k in ("tflops", "mfma_peak_frac", "stage_ms", "step_gpu_ms", "stage_pass_steps",
              "expert_counts", "roofline", "hbm_gbs_layer", "hbm_peak_frac_layer"):
        if k in h:
            rec[k] = h[k]
    if side:
        rec["workloads"] = {nm: r for nm, r in records.items() if nm != args.workload}

    if not args.no_cpu_baseline:
        T = args.tokens or moe_synth.WORKLOADS[args.workload].T
        sample = args.cpu_sample or min(T, 4096)
        log(f"[bench] timing the fp64 oracle on {sample} tokens")
        rec["cpu_baseline"] = cpu_baseline(args.workload, head_inputs, sample)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
