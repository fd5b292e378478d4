"""The library's host code under AddressSanitizer, on the CPU.

libmoe is rebuilt into a temporary directory with ASan on its host pass only
(the device code is unchanged; GPU sanitizers are not used) and the plain C
caller (tests/c_caller.c: sizes, status strings, argument validation, a
zero-token forward) runs against it with leak detection on and LIBMOE_LOG
set, so the validation paths and the call log are checked for out-of-bounds
accesses, use after free and leaks.  No call reaches the GPU."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_layer_gemv_amd", "csrc")
SOURCES = ["moe_api.cpp", "moe_router.hip", "moe_permute.hip", "moe_gemm.hip", "moe_decode.hip",
           "moe_combine.hip", "moe_stats.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# sanitizer flags for the host pass only: each -fsanitize= right after -Xarch_host
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_is_clean_under_asan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_ASAN,
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c",
                        os.path.join(CSRC, src), "-o", obj], check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = tmp_path / "libmoe.so"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_ASAN, *objs, "-o",
                    str(lib)], check=True, capture_output=True)
    exe = tmp_path / "c_caller"
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_caller.c"),
                    "-L", str(tmp_path), "-l:libmoe.so", f"-Wl,-rpath,{tmp_path}", "-o",
                    str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
                                LIBMOE_LOG="1"))
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
    assert "AddressSanitizer" not in r.stderr
    assert "libmoe: moe_forward" in r.stderr
