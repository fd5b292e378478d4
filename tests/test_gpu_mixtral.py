"""GPU parity at the full Mixtral shape (dim 4096, hidden 14336, 8 experts,
top-2; Table 1 of "Mixtral of Experts"), in the launch configuration the
benchmark times: decode (T=16), prefill (T=4096), skewed routing (T=4096,
~60% of slots on two experts) and a 32768-token batch fed as 4 chunks of 8192
through one reused workspace.

Routing (indices and gates) is checked for every token, and the layer output
element by element for every token: the fp64 oracle evaluates the batch in
blocks of 8192 tokens (the layer acts on each token independently, section
2.1), one expert at a time.
"""
import numpy as np
import pytest

import moe_synth
from oracle import moe_ref, parity
from tests.gpu_helpers import dev_bf16, host

pytestmark = pytest.mark.gpu

ORACLE_BLOCK = 8192


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_gemv_amd as m
    return m


@pytest.fixture(scope="module")
def mixtral_weights():
    w = moe_synth.WORKLOADS["prefill"]
    wg_f32, w1, w3, w2 = moe_synth.make_weights(w.weight_seed, w.D, w.H, w.n)
    d = dict(w1=dev_bf16(w1), w3=dev_bf16(w3), w2=dev_bf16(w2))
    return wg_f32, (w1, w3, w2), d


def oracle_full(x, wg, w1, w3, w2, K, forced_idx):
    """The oracle's output for every token, block by block."""
    T, D = x.shape
    y = np.empty((T, D))
    for c0 in range(0, T, ORACLE_BLOCK):
        c1 = min(T, c0 + ORACLE_BLOCK)
        y[c0:c1] = moe_ref.moe_layer(x[c0:c1], wg, w1, w3, w2, K,
                                     forced_idx=forced_idx[c0:c1])["y"]
    return y


def _run(moe, name, mixtral_weights, chunk=None):
    import torch
    w = moe_synth.WORKLOADS[name]
    wg_f32, (w1, w3, w2), d = mixtral_weights
    x = moe_synth.make_x(w.x_seed, w.T, w.D)
    wg = moe_synth.skew_gate(wg_f32, x, moe_synth.skew_coefficient()) if w.skew else moe_synth.bf16_bits(wg_f32)
    xd, wgd = dev_bf16(x), dev_bf16(wg)
    T, K = w.T, w.K
    chunk = chunk or T
    out = torch.empty((T, w.D), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(moe.workspace_bytes(moe.problem(chunk, w.D, w.H, w.n, K)), dtype=torch.uint8,
                     device="cuda:0")
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        moe.forward(xd[c0:c1], wgd, d["w1"], d["w3"], d["w2"], K, out=out[c0:c1],
                    topk_idx=idx[c0:c1], topk_gate=gate[c0:c1], workspace=ws)
    out_h, idx_h, gate_h = host(out), host(idx), host(gate)
    logits = moe_ref.router_logits(x, wg)
    rr = parity.check_routing(logits, K, idx_h, gate_h)
    counts = np.bincount(idx_h.ravel(), minlength=w.n)
    print(f"[{name}] routing: {rr} counts={counts.tolist()}")
    assert rr.ok, rr
    y_ref = oracle_full(x, wg, w1, w3, w2, K, rr.forced_idx)
    orep = parity.check_output(y_ref, out_h)
    print(f"[{name}] all {T} tokens: max/RMS={orep.max_rel:.3e} mean/RMS={orep.mean_rel:.3e}",
          flush=True)
    assert orep.ok, orep
    return counts


def test_decode_t16(moe, mixtral_weights):
    _run(moe, "decode", mixtral_weights)


@pytest.mark.parametrize("T", [1, 2, 4])
def test_decode_few_tokens(moe, mixtral_weights, T):
    # one to four tokens touch at most 2 to 8 experts: the weight-streaming
    # kernels split their contractions further to keep the chip busy
    import torch
    wg_f32, (w1, w3, w2), d = mixtral_weights
    w = moe_synth.WORKLOADS["decode"]
    x = moe_synth.make_x(w.x_seed, T, w.D)
    wg = moe_synth.bf16_bits(wg_f32)
    idx = torch.empty((T, 2), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    out = moe.forward(dev_bf16(x), dev_bf16(wg), d["w1"], d["w3"], d["w2"], 2, topk_idx=idx,
                      topk_gate=gate)
    rr = parity.check_routing(moe_ref.router_logits(x, wg), 2, host(idx), host(gate))
    assert rr.ok, rr
    ref = moe_ref.moe_layer(x, wg, w1, w3, w2, 2, forced_idx=rr.forced_idx)
    orep = parity.check_output(ref["y"], host(out))
    print(f"[decode T={T}] max/RMS={orep.max_rel:.3e} mean/RMS={orep.mean_rel:.3e}")
    assert orep.ok, orep


def test_prefill_t4096(moe, mixtral_weights):
    counts = _run(moe, "prefill", mixtral_weights)
    assert np.all(np.abs(counts / counts.sum() - 0.125) < 0.01)


def test_skewed_t4096(moe, mixtral_weights):
    counts = _run(moe, "skewed", mixtral_weights)
    assert abs(counts[:2].sum() / counts.sum() - 0.60) <= 0.01


def test_large_t32768_chunked(moe, mixtral_weights):
    _run(moe, "large", mixtral_weights, chunk=moe_synth.WORKLOADS["large"].chunk)
