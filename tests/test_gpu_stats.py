"""GPU routing diagnostics (moe_route_stats) against the oracle's exact counts
("Mixtral of Experts", section 5): random and structured choice arrays, dropped
ids, T = 0 and T = 1, n up to 256, and the router's own output on a Mixtral-shape
workload.  Integer counts: bit-exact."""
import numpy as np
import pytest

import moe_synth
from oracle import moe_ref
from tests.gpu_helpers import dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_gemv_amd as m
    return m


def _check(moe, idx, n):
    got = moe.route_stats(dev_i32(idx), n)
    want = moe_ref.route_stats(idx, n)
    for k in ("first", "any", "repeat_first", "repeat_either"):
        assert got[k] == want[k], (k, got[k], want[k])


CASES = [
    # T, K, n, seed, fraction of dropped ids
    (1, 2, 8, 1, 0.0),
    (2, 2, 8, 2, 0.0),
    (1000, 2, 8, 3, 0.0),
    (5000, 1, 8, 4, 0.0),
    (3001, 4, 16, 5, 0.0),
    (777, 3, 6, 6, 0.1),
    (4096, 2, 64, 7, 0.0),
    (9000, 8, 64, 8, 0.05),
    (4096, 8, 160, 9, 0.0),
    (3000, 6, 256, 10, 0.02),
]


@pytest.mark.parametrize("T,K,n,seed,drop", CASES)
def test_route_stats_random(moe, T, K, n, seed, drop):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(n, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    if drop:
        mask = rng.random(idx.shape) < drop
        idx[mask] = rng.choice([-1, n, n + 7], size=int(mask.sum()))
    _check(moe, idx, n)


def test_route_stats_structured_runs(moe):
    # long runs of the same experts: every consecutive pair repeats
    idx = np.repeat(np.array([[3, 5], [5, 3], [1, 2]], np.int32), 700, axis=0)
    _check(moe, idx, 8)


def test_route_stats_zero_tokens_writes_zeros(moe):
    import torch
    counts = torch.full((18,), 77, dtype=torch.int32, device="cuda:0")
    got = moe.route_stats(torch.empty((0, 2), dtype=torch.int32, device="cuda:0"), 8, counts=counts)
    assert got["first"] == [0] * 8 and got["any"] == [0] * 8
    assert got["repeat_first"] == 0 and got["repeat_either"] == 0


def test_route_stats_of_a_skewed_routing(moe):
    # the oracle's routing of the skewed Mixtral-shape workload (first 2048
    # tokens), fed to both sides
    x, wg = moe_synth.make_router_inputs("skewed")
    x = x[:2048]
    idx = moe_ref.topk_indices(moe_ref.router_logits(x, wg), 2).astype(np.int32)
    _check(moe, idx, 8)
    st = moe_ref.route_stats(idx, 8)
    assert 0.55 < (st["any"][0] + st["any"][1]) / idx.size < 0.65
