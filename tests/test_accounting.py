"""The benchmark's work accounting, checked against the parameter counts the
pages print for Mixtral 8x7B: 46.7B total (hackerpapers.qiaomu.ai digest) and
47B total / 13B active (the aipaper.jasonlin.tech abstract), from the Table 1
shapes of "Mixtral of Experts" section 2."""
import bench


def test_parameter_counts_match_the_pages():
    total, active = bench.mixtral_params()
    assert round(total / 1e9, 1) == 46.7
    assert round(total / 1e9) == 47 and round(active / 1e9) == 13


def test_layer_flops():
    # top-2 of 8 SwiGLU experts: 3 products of D x H per chosen expert
    assert bench.layer_flops(1, 4096, 14336, 8, 2) == 2 * 2 * 3 * 4096 * 14336 + 2 * 4096 * 8
    assert abs(bench.layer_flops(4096, 4096, 14336, 8, 2) / 1e12 - 2.8865) < 1e-4
    # the first product (w1 and w3) is two thirds of the expert work
    expert = bench.layer_flops(4096, 4096, 14336, 8, 2) - 2 * 4096 * 4096 * 8
    assert bench.up_flops(4096, 4096, 14336, 2) * 3 == expert * 2
