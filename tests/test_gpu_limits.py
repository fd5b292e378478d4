"""GPU parity at the largest batch the library accepts.

At dim 4096 the bound is T * D * 2 < 2^31 bytes of x, so T = 262143.  The
permuted layout then has 526336 rows, and the fp32 expert outputs
(rows x dim) hold more than 2^31 elements: any 32-bit element offset in the
expert products or the combine would wrap.  A narrow expert (hidden 64)
keeps the weights small; the expert-grouped GEMMs still run 2056 row tiles.

Routing (indices and gates) is checked for every token against the fp64
oracle's logits ("Mixtral of Experts", section 2.1, the G(x) and TopK
definitions); the layer output for a seeded sample of tokens spread over the
whole batch, the last ones included.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import moe_synth
from oracle import moe_ref, parity
from tests.gpu_helpers import dev_bf16, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_gemv_amd as m
    return m


def _x_parallel(seed, T, D):
    """make_x over [0, T), drawn block by block on worker threads (each block
    has its own child seed, so the values equal one make_x call)."""
    C = moe_synth.X_CHUNK
    starts = list(range(0, T, C))
    with ThreadPoolExecutor(max_workers=8) as pool:
        parts = list(pool.map(lambda s: moe_synth.make_x(seed, min(C, T - s), D, first_token=s),
                              starts))
    return np.concatenate(parts, axis=0)


def test_largest_batch_at_dim_4096(moe):
    import torch
    T, D, H, n, K = 262143, 4096, 64, 8, 2
    p = moe.problem(T, D, H, n, K)
    assert moe.workspace_bytes(moe.problem(T + 1, D, H, n, K)) == 0   # one token more is refused
    cap = moe.capacity_rows(p)
    assert cap * D > 2 ** 31
    seed = 41
    print(f"[limits] T={T} D={D} H={H} n={n} K={K} cap={cap}: generating", flush=True)
    x = _x_parallel(seed, T, D)
    wg_f32, w1, w3, w2 = moe_synth.make_weights(seed, D, H, n)
    wg = moe_synth.bf16_bits(wg_f32)
    out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    print(f"[limits] workspace {ws.numel() / 2**30:.1f} GiB; running moe_forward", flush=True)
    moe.forward(dev_bf16(x), dev_bf16(wg), dev_bf16(w1), dev_bf16(w3), dev_bf16(w2), K, out=out,
                topk_idx=idx, topk_gate=gate, workspace=ws)
    out_h, idx_h, gate_h = host(out), host(idx), host(gate)
    del ws, out
    print("[limits] checking routing", flush=True)
    logits = np.concatenate([moe_ref.router_logits(x[c:c + 32768], wg)
                             for c in range(0, T, 32768)])
    rr = parity.check_routing(logits, K, idx_h, gate_h)
    print(f"[limits] routing: {rr}", flush=True)
    assert rr.ok, rr
    rng = np.random.default_rng(seed)
    s = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T),
                                  rng.choice(T, size=56, replace=False)]))
    ref = moe_ref.moe_layer_rows(x[s], wg, w1, w3, w2, K, forced_idx=rr.forced_idx[s])
    orep = parity.check_output(ref["y"], out_h[s])
    print(f"[limits] sampled {s.size} tokens: max/RMS={orep.max_rel:.3e} "
          f"mean/RMS={orep.mean_rel:.3e}", flush=True)
    assert orep.ok, orep
