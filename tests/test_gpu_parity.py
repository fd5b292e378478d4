"""GPU parity of every libmoe entry point against the fp64 oracle, at sizes the
oracle finishes in seconds: several row/column/contraction tiles, ragged
tails, both expert paths (weight streaming for T <= 80 by default, up to 128
when forced; matrix-core tiles above), forced skewed and empty-expert routings, K and n variants,
and every router kernel (vector, one-launch matrix-core, slice kernel with either selection pass)."""
import numpy as np
import pytest

import moe_synth
from oracle import moe_ref, parity
from tests.gpu_helpers import dev_bf16, dev_i32, expected_permutation, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_gemv_amd as m
    return m


def _upload(L):
    return dict(x=dev_bf16(L.x), wg=dev_bf16(L.w_gate), w1=dev_bf16(L.w1), w3=dev_bf16(L.w3),
                w2=dev_bf16(L.w2))


def _check_forward(moe, L, label):
    import torch
    d = _upload(L)
    T, D, H, n, K = L.shape
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    out = moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], K, topk_idx=idx, topk_gate=gate)
    out_h, idx_h, gate_h = host(out), host(idx), host(gate)
    logits = moe_ref.router_logits(L.x, L.w_gate)
    rr = parity.check_routing(logits, K, idx_h, gate_h)
    print(f"[{label}] T={T} D={D} H={H} n={n} K={K} routing: {rr}")
    assert rr.ok, rr
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=rr.forced_idx)
    orep = parity.check_output(ref["y"], out_h)
    print(f"[{label}] output: max/RMS={orep.max_rel:.3e} mean/RMS={orep.mean_rel:.3e}")
    assert orep.ok, orep
    return d, out


SHAPES = [
    # label, T, D, H, n, K, seed
    ("tiny", 64, 128, 256, 8, 2, None),
    ("ragged_dims", 300, 200, 328, 8, 2, 11),
    ("multi_tile", 1500, 512, 768, 8, 2, 12),
    ("decode_t1", 1, 512, 1024, 8, 2, 13),
    ("decode_t2", 2, 256, 384, 8, 2, 14),
    ("decode_t16", 16, 512, 1024, 8, 2, 15),
    ("decode_t17", 17, 512, 1024, 8, 2, 16),
    ("decode_t32", 32, 384, 640, 8, 2, 17),
    # streaming with two row groups per lane (32 rows a pass) up to 64
    # tokens, four (64 rows) beyond, and the automatic threshold (80 tokens)
    # from both sides
    ("decode_t33", 33, 512, 1024, 8, 2, 18),
    ("decode_t48", 48, 512, 1024, 8, 2, 26),
    ("decode_t65", 65, 512, 1024, 8, 2, 27),
    ("decode_t80", 80, 512, 1024, 8, 2, 51),
    ("tiled_t81", 81, 512, 1024, 8, 2, 52),
    # wide experts (at least 32 column blocks): two column blocks per
    # first-product workgroup below T*K = 2.5n (9 tokens), four from there
    # (12, 24, 48 and 80 tokens: two, two, two and four row groups per lane),
    # then the tiled path
    ("stream_wide_t9", 9, 512, 4096, 8, 2, 54),
    ("stream_wide_t12", 12, 512, 4096, 8, 2, 46),
    ("stream_wide_t24", 24, 512, 4096, 8, 2, 47),
    ("stream_wide_t48", 48, 512, 4096, 8, 2, 48),
    ("stream_wide_t80", 80, 512, 4096, 8, 2, 49),
    ("tiled_wide_t81", 81, 512, 4096, 8, 2, 53),
    ("stream_wide_n16_t16", 16, 512, 4096, 16, 2, 50),
    # the tiled first product with its last round split along the contraction:
    # 8 experts x 112 column tiles = 896 tiles, 3 full rounds of 256 and a
    # half-full fourth whose 128 tiles run as 256 contraction halves
    ("tiled_split_t100", 100, 512, 14336, 8, 2, 55),
    ("k1_switch", 200, 256, 512, 8, 1, 19),
    ("n16_k4", 130, 256, 384, 16, 4, 20),
    ("n6_k3", 90, 136, 200, 6, 3, 21),
    ("n64_k2", 400, 128, 256, 64, 2, 22),
    # K = n: every expert on every token, the dense softmax mixture
    ("dense_k8", 300, 256, 384, 8, 8, 23),
    ("decode_dense_k8", 8, 256, 384, 8, 8, 24),
    ("k4_n32", 520, 256, 512, 32, 4, 25),
    # many small experts (the fine-grained layout): matrix-core router, up to
    # 256 experts, segments of a few rows each
    ("fine_n160_k8", 600, 256, 256, 160, 8, 28),
    ("fine_decode_t16", 16, 512, 256, 160, 8, 29),
    ("fine_decode_t1", 1, 256, 128, 160, 8, 34),
    ("n100_k6_ragged", 333, 200, 136, 100, 6, 30),
    ("n130_k5", 250, 136, 128, 130, 5, 32),
    ("n256_k8", 700, 384, 128, 256, 8, 31),
    ("n24_k3", 300, 256, 256, 24, 3, 35),
    # K = n = 96: slot selection runs past 64 slots per token
    ("dense_n96", 40, 128, 64, 96, 96, 33),
    # more tiles of the split second product than compute units, short
    # contractions (4 and 6 activation blocks per half)
    ("many_tiles_h256", 4096, 2048, 256, 8, 2, 36),
    ("many_tiles_h384", 4000, 2048, 384, 8, 2, 37),
    # split second product over more than one round of tiles, the last round
    # partly filled
    ("split_rounds", 2200, 2048, 1024, 8, 2, 38),
    # weight streaming with two column blocks per workgroup and the second
    # product's contraction in 4 partials (wide experts)
    ("stream_wide_split4", 16, 512, 4096, 8, 2, 39),
    # weight streaming with the first product's contraction in 2 partials
    # (narrow experts), added before silu * mul
    ("stream_narrow_up_split", 16, 2048, 256, 8, 2, 40),
    # the router's workgroup shape changes at 64 tokens (one token per
    # workgroup up to 64, four above); 16 experts at a decode-size batch
    ("router_t64", 64, 256, 384, 8, 2, 42),
    ("router_t65", 65, 256, 384, 8, 2, 43),
    ("decode_n16_k2", 24, 256, 384, 16, 2, 44),
    # the tiled products' shifted schedule (contractions of 8 + 12 r steps:
    # the first 8 as a straight-line head, then r whole rounds): 20 steps in
    # both products (dim 640; hidden 1280, two halves of 640), and 44 (dim
    # 1408; hidden 2816, two halves of 1408)
    ("shift_head_1_round", 300, 640, 1280, 8, 2, 56),
    ("shift_head_3_rounds", 300, 1408, 2816, 8, 2, 57),
    # one expert with 17 row tiles: cut into blocks of 9 and 8 row tiles in
    # the tiled products' tile order (an expert is cut from 16 row tiles on)
    ("one_expert_17_row_tiles", 4200, 256, 512, 1, 1, 45),
]


@pytest.mark.parametrize("label,T,D,H,n,K,seed", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_parity(moe, label, T, D, H, n, K, seed):
    if seed is None:
        L = moe_synth.make_workload("tiny")
    else:
        L = moe_synth.make_layer(T, D, H, n, K, seed=seed)
    _check_forward(moe, L, label)


def test_route_stage_and_logits(moe):
    import torch
    L = moe_synth.make_layer(777, 4096, 64, 8, 2, seed=31)
    d = _upload(L)
    T = 777
    logits = torch.empty((T, 8), dtype=torch.float32, device="cuda:0")
    idx, gate = moe.route(d["x"], d["wg"], 2, logits=logits)
    ref = moe_ref.router_logits(L.x, L.w_gate)
    lg = host(logits)
    # fp32 accumulation of 4096 products of magnitude ~1/64
    assert np.abs(lg - ref).max() < 2e-5
    rr = parity.check_routing(ref, 2, host(idx), host(gate))
    assert rr.ok, rr


@pytest.mark.parametrize("n,K,Ts", [
    (8, 2, (1, 63, 64, 65, 128, 1000, 5000, 9000)),
    # many experts; P = 72000 slots puts two 1024-slot rounds in a workgroup
    (160, 8, (1, 16, 127, 128, 4096, 9000)),
    (256, 4, (3, 600, 20000)),
], ids=["n8", "n160", "n256"])
def test_permute_stage_is_exact(moe, n, K, Ts):
    rng = np.random.default_rng(5 + n)
    for T in Ts:
        idx = np.stack([rng.choice(n, size=K, replace=False) for _ in range(T)]).astype(np.int32)
        p = moe.problem(T, 8, 8, n, K)
        cap = moe.capacity_rows(p)
        r = moe.permute(dev_i32(idx), n)
        cnt, off, rs, sr = expected_permutation(idx, n, moe.TILE_M, cap)
        assert np.array_equal(host(r["expert_count"]), cnt)
        assert np.array_equal(host(r["expert_offset"]), off)
        assert np.array_equal(host(r["row_slot"]), rs)
        assert np.array_equal(host(r["slot_row"]), sr)


# n % 64 == 0 gives the slowest (bank-conflicting) transposing reads of W_g:
# the case that shows a stage being refilled before every read of it is done
@pytest.mark.parametrize("n,D,T", [(8, 4096, 300), (8, 4096, 2048), (16, 512, 2500),
                                   (12, 256, 3000), (160, 4096, 300), (100, 1000, 300),
                                   (256, 512, 300), (128, 384, 700), (192, 384, 64),
                                   (192, 1024, 700), (224, 384, 200)])
def test_route_stage_logits_large_n(moe, n, D, T):
    import torch
    L = moe_synth.make_layer(T, D, 8, n, 8, seed=32 + n)
    x, wg = dev_bf16(L.x), dev_bf16(L.w_gate)
    logits = torch.empty((T, n), dtype=torch.float32, device="cuda:0")
    idx, gate = moe.route(x, wg, 8, logits=logits)
    ref = moe_ref.router_logits(L.x, L.w_gate)
    assert np.abs(host(logits) - ref).max() < 2e-5
    rr = parity.check_routing(ref, 8, host(idx), host(gate))
    assert rr.ok, rr


# Up to 16 experts (a multiple of 4) from 2048 tokens: router_fused_kernel
# while W_g, D rounded up to whole 32-row steps, fits its 64 KiB LDS copy
# (ragged token tail, D not a multiple of 32, exactly 64 KiB, two rounds of x
# steps per wave at D = 8192, K = n); beyond that the slice kernel and its
# selection pass (n = 16 at D = 4096, n = 8 at D = 8192)
@pytest.mark.parametrize("n,D,T,K", [(4, 4096, 2048, 1), (8, 4096, 4099, 2), (12, 1000, 2050, 3),
                                     (16, 2048, 2048, 4), (4, 8192, 2048, 2), (8, 512, 2048, 8),
                                     (16, 4096, 2048, 2), (8, 8192, 2100, 2)])
def test_route_matrix_core_paths_up_to_16_experts(moe, n, D, T, K):
    import torch
    L = moe_synth.make_layer(T, D, 8, n, K, seed=40 + n + D % 97)
    x, wg = dev_bf16(L.x), dev_bf16(L.w_gate)
    logits = torch.empty((T, n), dtype=torch.float32, device="cuda:0")
    idx, gate = moe.route(x, wg, K, logits=logits)
    ref = moe_ref.router_logits(L.x, L.w_gate)
    assert np.abs(host(logits) - ref).max() < 2e-5
    rr = parity.check_routing(ref, K, host(idx), host(gate))
    assert rr.ok, rr
    # without the optional logits output the choice and gates are the same
    idx2, gate2 = moe.route(x, wg, K)
    assert np.array_equal(host(idx2), host(idx)) and np.array_equal(host(gate2), host(gate))


def test_route_ties_go_to_the_lower_index_with_many_experts(moe):
    # W_g with duplicated columns gives exactly equal logits: the lower expert
    # index must win every tie, slot order by decreasing logit
    import torch
    D, n, K, T = 256, 160, 8, 40
    L = moe_synth.make_layer(T, D, 8, n, K, seed=77)
    wg = L.w_gate.copy()
    wg[:, 100:] = wg[:, :60]          # experts 100..159 copy experts 0..59
    idx, gate = moe.route(dev_bf16(L.x), dev_bf16(wg), K)
    ref = moe_ref.router_logits(L.x, wg)
    want = moe_ref.topk_indices(ref, K)
    assert np.array_equal(host(idx), want)


# T < 2048 takes the vector router (router_kernel), T >= 2048 the one-launch
# matrix-core router (router_fused_kernel) for n = 8
@pytest.mark.parametrize("T", [64, 1000, 2048, 4096])
def test_route_ties_go_to_the_lower_index_with_eight_experts(moe, T):
    # Mixtral's router shape (dim 4096, 8 experts, top-2) with W_g columns 5
    # and 7 copying columns 2 and 0: their logits are exactly equal, so every
    # tie the copies make must go to the lower index, with the slots in
    # decreasing-logit order, and two tied experts chosen together get equal
    # gates
    D, n, K = 4096, 8, 2
    L = moe_synth.make_layer(T, D, 8, n, K, seed=300 + T)
    wg = L.w_gate.copy()
    wg[:, 5] = wg[:, 2]
    wg[:, 7] = wg[:, 0]
    idx, gate = moe.route(dev_bf16(L.x), dev_bf16(wg), K)
    idx_h, gate_h = host(idx), host(gate)
    ref = moe_ref.router_logits(L.x, wg)
    want = moe_ref.topk_indices(ref, K)
    assert np.array_equal(idx_h, want)
    # ties decided here: a copy at the 2nd/3rd boundary lost to its original
    lost = ((want[:, 1] == 2) & ~np.any(want == 5, axis=1)) | \
           ((want[:, 1] == 0) & ~np.any(want == 7, axis=1))
    both = ((want[:, 0] == 2) & (want[:, 1] == 5)) | ((want[:, 0] == 0) & (want[:, 1] == 7))
    print(f"[ties n=8 T={T}] decided at the boundary: {int(lost.sum())}, "
          f"both copies chosen: {int(both.sum())}")
    assert lost.sum() > 0 and both.sum() > 0
    assert np.all(gate_h[both, 0] == gate_h[both, 1])
    rr = parity.check_routing(ref, K, idx_h, gate_h)
    assert rr.gate_max_err <= parity.GATE_TOL, rr


def test_permute_drops_out_of_range_experts(moe):
    idx = np.array([[0, 9], [-1, 3], [3, 0]], np.int32)
    r = moe.permute(dev_i32(idx), 8)
    sr = host(r["slot_row"])
    assert sr[1] == -1 and sr[2] == -1
    assert host(r["expert_count"]).tolist() == [2, 0, 0, 2, 0, 0, 0, 0]


FORCED = [
    # label, forced expert choice per token, T, D, H
    ("all_on_expert3", lambda T: np.tile([[3, 5]], (T, 1)), 700, 256, 384),
    ("counts_255_256_257", None, 0, 256, 384),
    ("one_expert_k1", lambda T: np.full((T, 1), 6), 600, 256, 384),
    # H = 1024: the second product runs as two contraction halves whose
    # partial sums are added before returning y_rows
    ("split_contraction", lambda T: np.stack([np.arange(T) % 8, (np.arange(T) + 3) % 8], 1), 900, 512, 1024),
    # two experts of 17 row tiles each: both cut into row blocks of 9 and 8 in
    # the tile order
    ("two_experts_17_row_tiles", lambda T: np.tile([[5, 2]], (T, 1)), 4200, 256, 384),
    # the tiled products cover an expert's rows with full 256-row tiles and
    # one tail tile of 64 rows (tail <= 64), 128 rows (<= 128) or 256 rows:
    # counts on both sides of every class boundary, with the second product's
    # contraction split in two (H = 1024)
    ("row_classes", None, 1, 512, 1024),
]


# The tiled first product's last-round split with one full round before it:
# 300 tokens on 12 of 16 experts (slots of token t on experts 2t and 2t + 1
# mod 12), 12 row tiles x 32 column tiles = 384 tiles = 256 + 128; the split
# halves' fp32 partials and the pass that adds them must give every slot's
# expert output.  (Forced tiling of one token at H = 1024 splits every tile:
# no full round, test_forced_expert_path.)
def test_grouped_ffn_split_last_round(moe):
    T, D, H, n, K = 300, 512, 4096, 16, 2
    t = np.arange(T)
    idx = np.stack([(2 * t) % 12, (2 * t + 1) % 12], 1).astype(np.int32)
    L = moe_synth.make_layer(T, D, H, n, K, seed=57)
    d = _upload(L)
    perm = moe.permute(dev_i32(idx), n)
    y_rows = moe.grouped_ffn(d["x"], perm["expert_count"], perm["expert_offset"], perm["row_slot"],
                             d["w1"], d["w3"], d["w2"], K, path=moe.PATH_TILED)
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=idx, return_slots=True)
    sr = host(perm["slot_row"])
    orep = parity.check_output(ref["E"], host(y_rows)[sr].reshape(T, K, D))
    print(f"[split last round] slots max/RMS={orep.max_rel:.3e} mean/RMS={orep.mean_rel:.3e}")
    assert orep.ok, orep


def _forced_counts_case():
    # expert 0: 255 slots, expert 1: 256, expert 2: 257, others empty (K=1)
    return np.concatenate([np.zeros(255), np.ones(256), np.full(257, 2)]).astype(np.int32)[:, None]


ROW_CLASS_COUNTS = [1, 63, 64, 65, 127, 128, 129, 256 + 64]


def _row_class_case():
    # K = 1, expert e holds ROW_CLASS_COUNTS[e] slots, tokens interleaved
    idx = np.concatenate([np.full(c, e) for e, c in enumerate(ROW_CLASS_COUNTS)])
    return np.random.default_rng(7).permutation(idx).astype(np.int32)[:, None]


@pytest.mark.parametrize("label,make,T,D,H", FORCED, ids=[f[0] for f in FORCED])
def test_grouped_ffn_forced_routing(moe, label, make, T, D, H):
    import torch
    if label == "row_classes":
        idx = _row_class_case()
    else:
        idx = _forced_counts_case() if make is None else np.asarray(make(T), np.int32)
    T, K = idx.shape
    n = 8
    L = moe_synth.make_layer(T, D, H, n, K, seed=41)
    d = _upload(L)
    perm = moe.permute(dev_i32(idx), n)
    y_rows = moe.grouped_ffn(d["x"], perm["expert_count"], perm["expert_offset"], perm["row_slot"],
                             d["w1"], d["w3"], d["w2"], K)
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=idx, return_slots=True)
    sr = host(perm["slot_row"])
    got = host(y_rows)[sr].reshape(T, K, D)
    orep = parity.check_output(ref["E"], got)
    print(f"[{label}] slots max/RMS={orep.max_rel:.3e} mean/RMS={orep.mean_rel:.3e}")
    assert orep.ok, orep
    # combine of the GPU's expert rows with the oracle's gates, against fp64
    gate = torch.from_numpy(ref["gate"].astype(np.float32)).to("cuda:0")
    out = moe.combine(y_rows, perm["slot_row"], gate)
    want = (ref["gate"].astype(np.float32).astype(np.float64)[:, :, None] * got).sum(axis=1)
    assert np.abs(host(out) - want).max() <= 1e-6 * np.abs(want).max()


# A caller's routing may name an expert more than once for one token: each
# slot is then its own row of that expert.  With every token of a 16-token
# batch on expert 3 twice (32 rows, more than one 16-row pass of the
# weight-streaming kernels) or thrice on expert 6 at T = 40 (120 rows, two
# passes of 64), both expert paths must compute every row.  With wide experts
# (H = 4096) the streaming first product forms h itself.
@pytest.mark.parametrize("T,K,H,path", [(16, 2, 1024, 1), (16, 2, 1024, 2), (40, 3, 1024, 1),
                                        (40, 3, 1024, 2), (16, 2, 4096, 1), (40, 3, 4096, 1)],
                         ids=["t16_k2_stream", "t16_k2_tiled", "t40_k3_stream", "t40_k3_tiled",
                              "t16_k2_stream_wide", "t40_k3_stream_wide"])
def test_grouped_ffn_repeated_expert_per_token(moe, T, K, H, path):
    D, n = 512, 8
    idx = np.zeros((T, K), np.int32)
    idx[:, :] = 3 if K == 2 else 6
    idx[::5, -1] = 1          # a few slots elsewhere
    L = moe_synth.make_layer(T, D, H, n, K, seed=420 + T + (0 if H == 1024 else 7))
    d = _upload(L)
    perm = moe.permute(dev_i32(idx), n)
    y_rows = moe.grouped_ffn(d["x"], perm["expert_count"], perm["expert_offset"], perm["row_slot"],
                             d["w1"], d["w3"], d["w2"], K, path=path)
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=idx, return_slots=True)
    sr = host(perm["slot_row"])
    assert np.all(sr >= 0)
    got = host(y_rows)[sr].reshape(T, K, D)
    orep = parity.check_output(ref["E"], got)
    print(f"[repeat T={T} K={K} path={path}] slots max/RMS={orep.max_rel:.3e} "
          f"mean/RMS={orep.mean_rel:.3e}")
    assert orep.ok, orep


# moe_grouped_ffn writes the rows that hold token-slots and leaves padding
# rows as they were, also when the second product's contraction is split and
# its partials are added afterwards (H = 1024 tiled at T = 900; wide experts
# streamed at T = 16, 4 partials, the first product forming h itself)
@pytest.mark.parametrize("T,D,H,path", [(900, 512, 1024, 2), (16, 512, 4096, 1)],
                         ids=["tiled_split", "stream_split4"])
def test_grouped_ffn_leaves_padding_rows(moe, T, D, H, path):
    import torch
    n, K = 8, 2
    L = moe_synth.make_layer(T, D, H, n, K, seed=430 + T)
    d = _upload(L)
    idx = moe_ref.topk_indices(moe_ref.router_logits(L.x, L.w_gate), K).astype(np.int32)
    perm = moe.permute(dev_i32(idx), n)
    cap = moe.capacity_rows(moe.problem(T, D, H, n, K))
    y_rows = torch.full((cap, D), 777.0, dtype=torch.float32, device="cuda:0")
    moe.grouped_ffn(d["x"], perm["expert_count"], perm["expert_offset"], perm["row_slot"],
                    d["w1"], d["w3"], d["w2"], K, y_rows=y_rows, path=path)
    y = host(y_rows)
    sr = host(perm["slot_row"])
    pad = np.ones(cap, bool)
    pad[sr] = False
    assert pad.sum() > 0
    assert np.all(y[pad] == 777.0)
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, K, forced_idx=idx, return_slots=True)
    orep = parity.check_output(ref["E"], y[sr].reshape(T, K, D))
    assert orep.ok, orep


# both expert-product paths: the tiled one combines permuted rows, the
# streaming one (automatic at 16 tokens, forced at 40) rows indexed by slot
@pytest.mark.parametrize("T,path", [(1000, 0), (16, 0), (40, 1), (24, 2)],
                         ids=["tiled", "stream", "stream_forced", "tiled_forced"])
def test_forward_is_deterministic_and_bf16_output_is_rne_of_fp32(moe, T, path):
    import torch
    L = moe_synth.make_layer(T, 512, 768, 8, 2, seed=51)
    d = _upload(L)
    run = lambda **kw: host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, path=path,
                                        **kw))
    a = run()
    b = run()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = run(out_dtype=moe.MOE_BF16)
    assert np.array_equal(c, moe_synth.bf16_bits(a))


def test_outputs_do_not_write_past_their_end(moe):
    import torch
    L = moe_synth.make_layer(100, 256, 384, 8, 2, seed=61)
    d = _upload(L)
    guard = 64
    out_buf = torch.full((100 * 256 + guard,), 12345.0, dtype=torch.float32, device="cuda:0")
    idx_buf = torch.full((200 + guard,), -777, dtype=torch.int32, device="cuda:0")
    gate_buf = torch.full((200 + guard,), 7.0, dtype=torch.float32, device="cuda:0")
    moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, out=out_buf[:25600].view(100, 256),
                topk_idx=idx_buf[:200].view(100, 2), topk_gate=gate_buf[:200].view(100, 2))
    assert np.all(host(out_buf)[25600:] == 12345.0)
    assert np.all(host(idx_buf)[200:] == -777)
    assert np.all(host(gate_buf)[200:] == 7.0)


def test_zero_tokens_is_a_noop(moe):
    import torch
    L = moe_synth.make_layer(4, 128, 256, 8, 2, seed=71)
    d = _upload(L)
    out = torch.empty((0, 128), dtype=torch.float32, device="cuda:0")
    moe.forward(d["x"][:0], d["wg"], d["w1"], d["w3"], d["w2"], 2, out=out,
                workspace=torch.empty(256, dtype=torch.uint8, device="cuda:0"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,path", [(16, 2), (1, 2), (32, 2), (96, 1), (128, 1), (113, 1)],
                         ids=["tiled_t16", "tiled_t1", "tiled_t32", "stream_t96", "stream_t128",
                              "stream_t113"])
def test_forced_expert_path(moe, T, path):
    # both expert-product paths at batch sizes where the other one is the default
    L = moe_synth.make_layer(T, 512, 1024, 8, 2, seed=90 + T)
    d = _upload(L)
    out = moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, path=path)
    logits = moe_ref.router_logits(L.x, L.w_gate)
    import torch
    idx = torch.empty((T, 2), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, 2), dtype=torch.float32, device="cuda:0")
    moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, topk_idx=idx, topk_gate=gate, path=path)
    rr = parity.check_routing(logits, 2, host(idx), host(gate))
    assert rr.ok, rr
    ref = moe_ref.moe_layer(L.x, L.w_gate, L.w1, L.w3, L.w2, 2, forced_idx=rr.forced_idx)
    orep = parity.check_output(ref["y"], host(out))
    assert orep.ok, orep


@pytest.mark.parametrize("path,H", [(1, 1024), (2, 1024), (1, 4096)],
                         ids=["stream", "tiled", "stream_wide"])
def test_every_token_on_the_same_two_experts(moe, path, H):
    # 64 copies of one token row: every token routes to the same two experts,
    # so each of them holds all 64 slots (the most the streaming path takes
    # per expert, in two row passes); every output row must equal the
    # oracle's single-token result
    import dataclasses
    L = moe_synth.make_layer(64, 512, H, 8, 2, seed=95)
    L = dataclasses.replace(L, x=np.repeat(L.x[:1], 64, axis=0))
    d = _upload(L)
    import torch
    idx = torch.empty((64, 2), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((64, 2), dtype=torch.float32, device="cuda:0")
    out = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, topk_idx=idx,
                           topk_gate=gate, path=path))
    idx_h = host(idx)
    assert (idx_h == idx_h[:1]).all() and len(set(idx_h[0].tolist())) == 2
    logits = moe_ref.router_logits(L.x[:1], L.w_gate)
    rr = parity.check_routing(logits, 2, idx_h[:1], host(gate)[:1])
    assert rr.ok, rr
    ref = moe_ref.moe_layer(L.x[:1], L.w_gate, L.w1, L.w3, L.w2, 2, forced_idx=rr.forced_idx)
    orep = parity.check_output(np.repeat(ref["y"], 64, axis=0), out)
    assert orep.ok, orep
    # identical tokens give identical rows, bit for bit
    assert np.array_equal(out.view(np.uint32), np.repeat(out[:1], 64, axis=0).view(np.uint32))


def test_stream_path_rejects_large_batches(moe):
    import torch
    T = moe.STREAM_MAX_TOKENS + 1
    L = moe_synth.make_layer(T, 128, 256, 8, 2, seed=99)
    d = _upload(L)
    # a workspace the tiled path would take: the refusal is the path's limit
    ws = torch.empty(moe.workspace_bytes(moe.problem(T, 128, 256, 8, 2)), dtype=torch.uint8,
                     device="cuda:0")
    with pytest.raises(moe.MoeError) as err:
        moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, path=moe.PATH_STREAM,
                    workspace=ws)
    assert err.value.status == moe.MOE_ENOTSUP


@pytest.mark.parametrize("T,D,H,n,K", [(300, 256, 384, 8, 2), (16, 512, 1024, 8, 2),
                                       (200, 256, 256, 160, 8)],
                         ids=["tiled", "streaming", "n160_matrix_router"])
def test_forward_graph_capture_replays_match_eager(moe, T, D, H, n, K):
    # Every stage only enqueues kernels on the caller's stream (no host reads,
    # no allocation, no memset nodes), so moe_forward can be captured into a
    # HIP graph.  Each replay, with eager work and synchronisation between
    # replays, must give the eager result bit for bit.
    import torch
    L = moe_synth.make_layer(T, D, H, n, K, seed=300 + T)
    d = _upload(L)
    p = moe.problem(T, D, H, n, K)
    ws = torch.empty(moe.workspace_bytes(p), dtype=torch.uint8, device="cuda:0")
    args = (d["x"], d["wg"], d["w1"], d["w3"], d["w2"], K)
    eager = host(moe.forward(*args, workspace=ws)).copy()
    out = torch.empty((T, D), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda:0")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as torch asks before capture
        moe.forward(*args, out=out, topk_idx=idx, topk_gate=gate, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(*args, out=out, topk_idx=idx, topk_gate=gate, workspace=ws)
    for r in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xAB)          # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(out)
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {r}"


def test_concurrent_streams_with_separate_workspaces(moe):
    # Calls that may overlap need separate workspaces; with them, a tiled and a
    # weight-streaming forward enqueued on two streams at once (each a few
    # times, interleaved) give their one-stream results bit for bit.
    import torch
    layers = [moe_synth.make_layer(300, 256, 1024, 8, 2, seed=410),
              moe_synth.make_layer(16, 512, 1024, 8, 2, seed=411)]
    runs = []
    for L in layers:
        T, D, H, n, K = L.shape
        d = _upload(L)
        ws = torch.empty(moe.workspace_bytes(moe.problem(T, D, H, n, K)), dtype=torch.uint8,
                         device="cuda:0")
        args = (d["x"], d["wg"], d["w1"], d["w3"], d["w2"], K)
        ref = host(moe.forward(*args, workspace=ws)).copy()
        outs = [torch.full((T, D), float("nan"), device="cuda:0") for _ in range(3)]
        runs.append((args, ws, ref, outs))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for (args, ws, _, outs), s_ in zip(runs, streams):
            with torch.cuda.stream(s_):
                moe.forward(*args, out=outs[rep], workspace=ws)
    torch.cuda.synchronize()
    for i, (_, _, ref, outs) in enumerate(runs):
        for rep, o in enumerate(outs):
            assert np.array_equal(host(o).view(np.uint32), ref.view(np.uint32)), (i, rep)


@pytest.mark.parametrize("T,D,H,n,K", [(300, 256, 1024, 8, 2), (16, 512, 1024, 8, 2),
                                       (200, 256, 256, 160, 8), (16, 512, 4096, 8, 2),
                                       (16, 2048, 256, 8, 2)],
                         ids=["tiled_split", "streaming_split", "n160", "streaming_split4",
                              "streaming_up_split"])
def test_stage_chain_matches_forward(moe, T, D, H, n, K):
    # moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine gives moe_forward's
    # output bit for bit (the stage path adds the split partials before the
    # combine, the fused path inside it, in the same order)
    import torch
    L = moe_synth.make_layer(T, D, H, n, K, seed=400 + T)
    d = _upload(L)
    fwd = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], K)).copy()
    idx, gate = moe.route(d["x"], d["wg"], K)
    perm = moe.permute(idx, n)
    y_rows = moe.grouped_ffn(d["x"], perm["expert_count"], perm["expert_offset"], perm["row_slot"],
                             d["w1"], d["w3"], d["w2"], K)
    out = host(moe.combine(y_rows, perm["slot_row"], gate))
    assert np.array_equal(out.view(np.uint32), fwd.view(np.uint32))


def test_forward_timed_events_bracket_the_stages(moe):
    # moe_forward_timed: same result as moe_forward, and the 6 events it records
    # are ordered, so the stage times are non-negative and add up
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(6):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    L = moe_synth.make_layer(500, 256, 512, 8, 2, seed=501)
    d = _upload(L)
    a = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2)).copy()
    b = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, events=evs)).copy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ms = []
    for i in range(5):
        t = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(evs[i]),
                                       ctypes.c_void_p(evs[i + 1])) == 0
        ms.append(t.value)
    total = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(total), ctypes.c_void_p(evs[0]),
                                   ctypes.c_void_p(evs[5])) == 0
    assert all(m >= 0 for m in ms)
    assert abs(sum(ms) - total.value) <= 1e-3 + 1e-3 * total.value
    # null entries are skipped: only the two around the first expert product,
    # on the tiled and on the weight-streaming path (which has no permute pass)
    for T in (500, 16):
        L = moe_synth.make_layer(T, 256, 512, 8, 2, seed=502 + T)
        d = _upload(L)
        a = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2)).copy()
        part = [None, None, evs[2], evs[3], None, None]
        b = host(moe.forward(d["x"], d["wg"], d["w1"], d["w3"], d["w2"], 2, events=part)).copy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        t = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(evs[2]),
                                       ctypes.c_void_p(evs[3])) == 0
        assert t.value > 0
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
