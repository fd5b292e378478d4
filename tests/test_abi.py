"""The libmoe C ABI on the CPU: the library loads, exports every function that
include/libmoe.h declares, and rejects bad arguments before touching the GPU.
No call here reaches a kernel launch (tokens == 0 returns before any HIP call,
and every other call fails validation)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")


@pytest.fixture(scope="module")
def moe():
    lib_path = os.path.join(ROOT, "sparse_moe_layer_gemv_amd", "libmoe.so")
    if not os.path.exists(lib_path):
        import runpy
        runpy.run_path(os.path.join(ROOT, "sparse_moe_layer_gemv_amd", "_build.py"))["build"]()
    import sparse_moe_layer_gemv_amd as m
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for f in ("moe_route", "moe_route_workspace_bytes", "moe_permute", "moe_grouped_ffn",
              "moe_combine", "moe_forward",
              "moe_workspace_bytes", "moe_capacity_rows", "moe_status_string",
              "moe_decode_max_tokens"):
        assert f in names


def test_binding_constants_match_the_header(moe):
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (MOE_[A-Z_]+) \(?([0-9u* ]+)\)?", text))
    val = lambda k: eval(defs[k].replace("u", ""))
    assert val("MOE_TILE_M") == moe.TILE_M
    assert val("MOE_MAX_EXPERTS") == moe.MAX_EXPERTS
    assert val("MOE_STREAM_MAX_TOKENS") == moe.STREAM_MAX_TOKENS
    assert val("MOE_NOALLOC_SCRATCH_BYTES") == moe.NOALLOC_SCRATCH_BYTES


def test_library_exports_every_declared_symbol(moe):
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(moe.lib, name)
    assert set(moe.EXPORTED) == set(_declared_functions())


def test_capacity_and_workspace(moe):
    p = moe.problem(4096, 4096, 14336, 8, 2)
    cap = moe.capacity_rows(p)
    assert cap == ((8192 + 8 * 255 + 255) // 256) * 256
    ws = moe.workspace_bytes(p)
    # h (bf16) and two fp32 partials of y_rows dominate
    assert ws >= cap * (14336 * 2 + 2 * 4096 * 4)
    assert ws < cap * (14336 * 2 + 2 * 4096 * 4) + 4 * 1024 * 1024
    assert moe.capacity_rows(moe.problem(4096, 4096, 14336, 8, 9)) == -1   # K > n
    assert moe.workspace_bytes(moe.problem(16, 4100, 14336, 8, 2)) == 0    # dim % 8
    assert moe.workspace_bytes(moe.problem(16, 4096, 14336, 257, 2)) == 0  # n > 256
    assert moe.workspace_bytes(moe.problem(16, 4096, 768, 256, 8)) > 0     # n = 256
    # sizes past the kernels' 32-bit byte offsets are refused, the largest below them accepted
    assert moe.workspace_bytes(moe.problem(262144, 4096, 64, 8, 2)) == 0    # T*D*2 = 2^31
    assert moe.workspace_bytes(moe.problem(262143, 4096, 64, 8, 2)) > 0
    assert moe.workspace_bytes(moe.problem(4, 16, 1 << 26, 8, 2)) == 0      # D*H*2 = 2^31
    assert moe.workspace_bytes(moe.problem(4, 8, 1 << 22, 8, 2)) == 0       # 256*H*2 = 2^31
    assert moe.workspace_bytes(moe.problem(4, 8, (1 << 22) - 8, 8, 2)) > 0
    assert moe.decode_max_tokens() >= 16
    # expert-product path: unknown values are invalid; forced streaming only up
    # to STREAM_MAX_TOKENS; its scratch is part of the workspace
    assert moe.workspace_bytes(moe.problem(16, 4096, 14336, 8, 2, path=3)) == 0
    assert moe.decode_max_tokens() <= moe.STREAM_MAX_TOKENS
    assert moe.workspace_bytes(moe.problem(moe.STREAM_MAX_TOKENS, 4096, 14336, 8, 2,
                                           path=moe.PATH_STREAM)) > 0
    big = moe.STREAM_MAX_TOKENS + 1
    assert moe.workspace_bytes(moe.problem(big, 4096, 14336, 8, 2, path=moe.PATH_STREAM)) == 0
    assert moe.workspace_bytes(moe.problem(big, 4096, 14336, 8, 2, path=moe.PATH_TILED)) > 0
    assert moe.workspace_bytes(moe.problem(16, 4096, 14336, 8, 2, path=moe.PATH_STREAM)) >= \
        2 * 16 * 2 * 14336 * 4


def test_status_strings(moe):
    for s in range(5):
        assert moe.lib.moe_status_string(s)
    assert moe.lib.moe_status_string(99) == b"unknown status"


FAKE = 0x100000  # a 256-byte-aligned non-null address; validation never dereferences it


def _fwd(moe, p, ptrs=None, ws=FAKE, ws_bytes=None):
    ptrs = ptrs or {}
    args = [ptrs.get(k, FAKE) for k in ("x", "wg", "w1", "w3", "w2", "out")]
    if ws_bytes is None:
        ws_bytes = moe.workspace_bytes(p)
    return moe.lib.moe_forward(ctypes.byref(p), *args, None, None, ws, ws_bytes, None)


def test_validation_errors(moe):
    good = moe.problem(64, 128, 256, 8, 2)
    assert _fwd(moe, moe.problem(0, 128, 256, 8, 2)) == moe.MOE_OK          # T = 0: no-op
    assert _fwd(moe, moe.problem(-1, 128, 256, 8, 2)) == moe.MOE_EINVAL
    assert _fwd(moe, moe.problem(64, 128, 256, 8, 0)) == moe.MOE_EINVAL     # K < 1
    assert _fwd(moe, moe.problem(64, 128, 256, 8, 9)) == moe.MOE_EINVAL     # K > n
    assert _fwd(moe, moe.problem(64, 130, 256, 8, 2)) == moe.MOE_EINVAL     # dim % 8
    assert _fwd(moe, moe.problem(64, 128, 250, 8, 2)) == moe.MOE_EINVAL     # hidden % 8
    assert _fwd(moe, moe.problem(64, 128, 256, 257, 2)) == moe.MOE_ENOTSUP  # n > 256
    assert _fwd(moe, moe.problem(64, 128, 256, 8, 2, 7)) == moe.MOE_EINVAL  # out dtype
    assert _fwd(moe, good, {"x": 0}) == moe.MOE_EINVAL                      # null
    assert _fwd(moe, good, {"w1": FAKE + 8}) == moe.MOE_EINVAL              # misaligned
    assert _fwd(moe, good, ws=0) == moe.MOE_EWORKSPACE
    assert _fwd(moe, good, ws_bytes=moe.workspace_bytes(good) - 1) == moe.MOE_EWORKSPACE
    assert _fwd(moe, good, ws=FAKE + 16) == moe.MOE_EINVAL                  # ws not 256-aligned
    assert moe.lib.moe_forward(None, *([FAKE] * 6), None, None, FAKE, 1 << 30, None) == moe.MOE_EINVAL


def test_stage_validation_errors(moe):
    p = moe.problem(64, 128, 256, 8, 2)
    L = moe.lib
    assert L.moe_route(ctypes.byref(p), 0, FAKE, FAKE, FAKE, None, None, 0, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE + 4, None, 0,
                       None) == moe.MOE_EINVAL
    # more than 16 experts: the matrix-core router needs its scratch
    q = moe.problem(64, 128, 256, 160, 8)
    assert moe.route_workspace_bytes(q) > 0
    assert moe.route_workspace_bytes(p) == 0
    assert L.moe_route(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, None, None, 0,
                       None) == moe.MOE_EWORKSPACE
    assert L.moe_route(ctypes.byref(q), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                       moe.route_workspace_bytes(q) - 1, None) == moe.MOE_EWORKSPACE
    assert L.moe_permute(ctypes.byref(p), FAKE, FAKE, FAKE, 0, FAKE, None) == moe.MOE_EINVAL
    assert L.moe_grouped_ffn(ctypes.byref(p), *([FAKE] * 8), FAKE, 16, None) == moe.MOE_EWORKSPACE
    assert L.moe_combine(ctypes.byref(p), FAKE, FAKE, FAKE, 0, None) == moe.MOE_EINVAL
    z = moe.problem(0, 128, 256, 8, 2)
    assert L.moe_route(ctypes.byref(z), 0, 0, 0, 0, None, None, 0, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(z), 0, 0, 0, 0, None) == moe.MOE_OK


def test_noalloc_refuses_before_any_device_call(moe):
    # Refusals of moe_forward_noalloc come from the host checks alone, before
    # the device is touched, so they hold here without a GPU: the tiled path,
    # a batch the automatic choice tiles, and intermediates larger than the
    # array.  64 tokens of 262144-wide experts need at least T*K*H bf16 values
    # of h, twice the array.
    L = moe.lib

    def call(p):
        return L.moe_forward_noalloc(ctypes.byref(p), *([FAKE] * 6), None, None, None)

    assert call(moe.problem(16, 512, 1024, 8, 2, path=moe.PATH_TILED)) == moe.MOE_ENOTSUP
    assert call(moe.problem(moe.decode_max_tokens() + 1, 512, 1024, 8, 2)) == moe.MOE_ENOTSUP
    assert 64 * 2 * 262144 * 2 >= 2 * moe.NOALLOC_SCRATCH_BYTES
    assert call(moe.problem(64, 1024, 262144, 8, 2, path=moe.PATH_STREAM)) == moe.MOE_ENOTSUP


def test_binding_rejects_cpu_tensors(moe):
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.route(x, torch.zeros((128, 8), dtype=torch.bfloat16), 2,
                  topk_idx=torch.zeros((4, 2), dtype=torch.int32),
                  topk_gate=torch.zeros((4, 2)))


def test_libmoe_log_prints_one_line_per_call(moe):
    # LIBMOE_LOG in a child process: a valid zero-token forward (no GPU work)
    # and an invalid one (K > n) each print one line with the status; without
    # the variable nothing is printed
    code = (
        "import ctypes, sparse_moe_layer_gemv_amd as m\n"
        "p = m.problem(0, 512, 1024, 8, 2)\n"
        "q = m.problem(16, 512, 1024, 8, 9)\n"
        "print(m.lib.moe_forward(ctypes.byref(p), None, None, None, None, None, None, None,"
        " None, None, 0, None))\n"
        "print(m.lib.moe_forward(ctypes.byref(q), None, None, None, None, None, None, None,"
        " None, None, 0, None))\n")
    env = dict(os.environ, PYTHONPATH=ROOT)
    on = subprocess.run(["python3", "-c", code], capture_output=True, text=True, cwd=ROOT,
                        env=dict(env, LIBMOE_LOG="1"), timeout=300)
    assert on.returncode == 0, on.stderr
    assert on.stdout.split() == [str(moe.MOE_OK), str(moe.MOE_EINVAL)]
    lines = [l for l in on.stderr.splitlines() if l.startswith("libmoe: ")]
    assert lines == [
        "libmoe: moe_forward T=0 D=512 H=1024 n=8 K=2 out=f32 path=stream -> 0 (ok)",
        "libmoe: moe_forward T=16 D=512 H=1024 n=8 K=9 out=f32 path=- -> 1 (invalid argument)",
    ]
    off = subprocess.run(["python3", "-c", code], capture_output=True, text=True, cwd=ROOT,
                         env=dict(env, LIBMOE_LOG="0"), timeout=300)
    assert off.returncode == 0, off.stderr
    assert not [l for l in off.stderr.splitlines() if l.startswith("libmoe: ")]
