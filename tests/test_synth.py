"""The seeded input generator (CPU only): determinism, bf16 rounding, and the
routing statistics of the Mixtral-shape workloads measured with the oracle."""
import numpy as np
import pytest

import moe_synth
from oracle import moe_ref


def test_bf16_round_to_nearest_even_edges():
    f = np.array([
        1.0,                      # exact
        1.0 + 2.0 ** -8,          # halfway between 1 and 1+2^-7 -> ties to even (1.0)
        1.0 + 3 * 2.0 ** -8,      # halfway, odd below -> rounds up to 1+2^-6
        1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above halfway -> up
        -0.0, 0.0, np.inf, -np.inf,
        1e-40,                    # float32 subnormal
        3.4028235e38,             # max float32 rounds to inf in bf16
    ], dtype=np.float32)
    got = moe_synth.bf16_bits(f).tolist()
    assert got == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x8000, 0x0000, 0x7F80, 0xFF80, 0x0001, 0x7F80]
    nan = moe_synth.bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bf16_roundtrip_exact_on_bf16_values():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = moe_synth.bf16_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(moe_synth.bf16_bits(f[finite]), bits[finite])


def test_generator_is_deterministic_and_chunked():
    a = moe_synth.make_layer(70, 32, 48, 8, 2, seed=77)
    b = moe_synth.make_layer(70, 32, 48, 8, 2, seed=77)
    for name in ("x", "w_gate", "w1", "w3", "w2"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    # any token range equals the corresponding slice of the full sequence
    full = moe_synth.make_x(5, 8192 + 200, 16)
    part = moe_synth.make_x(5, 200, 16, first_token=8100)
    assert np.array_equal(full[8100:8300], part)


def test_distributions():
    L = moe_synth.make_layer(2048, 256, 512, 8, 2, seed=3)
    x = moe_synth.bf16_to_f32(L.x)
    assert abs(x.std() - 1.0) < 0.01 and abs(x.mean()) < 0.01
    w1 = moe_synth.bf16_to_f32(L.w1)
    assert abs(w1.std() * np.sqrt(256) - 1.0) < 0.01
    w2 = moe_synth.bf16_to_f32(L.w2)
    assert abs(w2.std() * np.sqrt(512) - 1.0) < 0.01


@pytest.mark.slow
def test_prefill_routing_is_balanced():
    # Figure 7 of section 5 marks 1/8 as the share under uniform assignment
    x, wg = moe_synth.make_router_inputs("prefill")
    idx = moe_ref.topk_indices(moe_ref.router_logits(x, wg), 2)
    share = moe_ref.expert_share(idx, 8)
    assert np.all(np.abs(share - 0.125) < 0.01), share
    first, either = moe_ref.consecutive_repeat(idx)
    # Table 5 closed forms 1/8 and 1-(6/8)(5/7); sigma ~0.5% at 4095 pairs
    assert abs(first - 0.125) < 0.025 and abs(either - 0.4643) < 0.04


@pytest.mark.slow
def test_skewed_routing_share_is_calibrated():
    x, wg = moe_synth.make_router_inputs("skewed")
    idx = moe_ref.topk_indices(moe_ref.router_logits(x, wg), 2)
    share = moe_ref.expert_share(idx, 8)
    assert abs(share[:2].sum() - 0.60) <= 0.01, share
