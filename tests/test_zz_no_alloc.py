"""moe_forward_noalloc, the workspace-free form of moe_forward for callers that
cannot allocate device memory, through the C ABI: two calls in a row (the
second on a smaller batch, so it runs over what the first left in the
library's array) must give moe_forward's results bit for bit, and the
oracle's within the layer tolerances; shapes beyond the array, and the tiled
path, are refused before anything is enqueued."""
import ctypes

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


def _layer(moe, L, T, fn):
    import torch
    _, D, H, n, K = L.shape
    x = dev_bf16(L.x[:T])
    w = [dev_bf16(a) for a in (L.w_gate, L.w1, L.w3, L.w2)]
    out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    fn(x, *w, K, out=out, topk_idx=idx, topk_gate=gate)
    return host(out), host(idx), host(gate)


# (label, first T, second T, D, H, n, K, path): Mixtral-like 8 experts top-2
# on the vector router; 160 experts top-8 on the matrix-core router (its
# partial logits in the array too) with the first product's contraction
# split; the forced streaming path at 64 tokens with wide experts (the
# second product in 4 partials)
CASES = [
    ("n8_k2", 32, 7, 1024, 2048, 8, 2, 0),
    ("n160_k8", 16, 3, 2048, 256, 160, 8, 0),
    ("stream_t64_wide", 64, 33, 512, 4096, 8, 2, 1),
]


@pytest.mark.parametrize("label,T1,T2,D,H,n,K,path", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_forward(moe, label, T1, T2, D, H, n, K, path):
    L = moe_synth.make_layer(T1, D, H, n, K, seed=500 + n)
    for T in (T1, T2):
        print(f"[noalloc {label}] T={T} D={D} H={H} n={n} K={K} path={path}", flush=True)
        ref_out, ref_idx, ref_gate = _layer(
            moe, L, T, lambda *a, **k: moe.forward(*a, **k, path=path))
        out, idx, gate = _layer(moe, L, T, lambda *a, **k: moe.forward_noalloc(*a, **k, path=path))
        assert np.array_equal(idx, ref_idx)
        assert np.array_equal(gate.view(np.uint32), ref_gate.view(np.uint32))
        assert np.array_equal(out.view(np.uint32), ref_out.view(np.uint32))
        logits = moe_ref.router_logits(L.x[:T], L.w_gate)
        rr = parity.check_routing(logits, K, idx, gate)
        assert rr.ok, rr
        y = moe_ref.moe_layer(L.x[:T], L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=rr.forced_idx)["y"]
        orep = parity.check_output(y, out)
        assert orep.ok, orep
        # bf16 output: the same fp32 sums, rounded to nearest even
        import torch
        ob = torch.empty((T, D), dtype=torch.bfloat16, device="cuda:0")
        w = [dev_bf16(a) for a in (L.w_gate, L.w1, L.w3, L.w2)]
        moe.forward_noalloc(dev_bf16(L.x[:T]), *w, K, out=ob, out_dtype=moe.MOE_BF16, path=path)
        assert np.array_equal(host(ob), moe_synth.bf16_bits(out))


def test_noalloc_refuses_what_does_not_fit(moe):
    import torch
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda:0")
    ptr = buf.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream

    def call(T, D, H, n, K, path=0):
        p = moe.problem(T, D, H, n, K, path=path)
        return moe.lib.moe_forward_noalloc(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, None,
                                           None, stream)

    # the tiled path, a batch the automatic choice tiles, and intermediates
    # beyond the array are refused with nothing launched: the buffer stays
    # zero.  64 tokens of 262144-wide experts need at least T*K*H bf16 values
    # of h (the smallest form any first product writes), 64 MiB: checked here
    # before the call, since an accepted call would run the layer on the
    # 64 KiB buffer
    assert call(16, 512, 1024, 8, 2, path=moe.PATH_TILED) == moe.MOE_ENOTSUP
    assert call(moe.decode_max_tokens() + 1, 512, 1024, 8, 2) == moe.MOE_ENOTSUP
    T, D, H, K = 64, 1024, 262144, 2
    assert T * K * H * 2 >= 2 * moe.NOALLOC_SCRATCH_BYTES
    assert call(T, D, H, 8, K, path=moe.PATH_STREAM) == moe.MOE_ENOTSUP
    assert call(0, 512, 1024, 8, 2) == moe.MOE_OK
    torch.cuda.synchronize()
    assert int(buf.count_nonzero()) == 0
