"""Python binding of libmoe, the Mixtral sparse MoE layer on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/libmoe.h``: every
function takes PyTorch tensors only as holders of device memory, checks their
dtype/shape/device, and passes raw pointers plus the current HIP stream.  All
arithmetic runs in the HIP kernels of ``libmoe.so``; there is no fallback.

Importing this package fails loudly if ``libmoe.so`` has not been built
(``python sparse_moe_layer_gemv_amd/_build.py``).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

_HINT = "build it with `python sparse_moe_layer_gemv_amd/_build.py` (hipcc, gfx950)"
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmoe.so not found at {LIB_PATH}; {_HINT}")

lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 2
TILE_M = 256
MAX_EXPERTS = 256
STREAM_MAX_TOKENS = 128
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024

EXPORTED = ("moe_capacity_rows", "moe_workspace_bytes", "moe_status_string", "moe_route",
            "moe_route_workspace_bytes",
            "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
            "moe_decode_max_tokens", "moe_forward_timed", "moe_route_stats",
            "moe_forward_noalloc")


for _name in EXPORTED:
    if not hasattr(lib, _name):
        raise ImportError(f"{LIB_PATH} lacks {_name} (stale build); {_HINT}")


class Problem(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("dim", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("path", ctypes.c_int32)]


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
lib.moe_capacity_rows.argtypes = [_P]
lib.moe_capacity_rows.restype = ctypes.c_int64
lib.moe_workspace_bytes.argtypes = [_P]
lib.moe_workspace_bytes.restype = ctypes.c_size_t
lib.moe_status_string.argtypes = [ctypes.c_int32]
lib.moe_status_string.restype = ctypes.c_char_p
lib.moe_decode_max_tokens.argtypes = []
lib.moe_decode_max_tokens.restype = ctypes.c_int32
lib.moe_route_workspace_bytes.argtypes = [_P]
lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
lib.moe_route.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.moe_permute.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp]
lib.moe_grouped_ffn.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.moe_combine.argtypes = [_P, _vp, _vp, _vp, _vp, _vp]
lib.moe_route_stats.argtypes = [_P, _vp, _vp, _vp]
lib.moe_forward.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
lib.moe_forward_timed.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                  _vp, ctypes.POINTER(_vp)]
lib.moe_forward_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
for _f in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
           "moe_forward_timed", "moe_route_stats", "moe_forward_noalloc"):
    getattr(lib, _f).restype = ctypes.c_int32


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib.moe_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def problem(tokens: int, dim: int, hidden: int, n_experts: int, top_k: int,
            out_dtype: int = MOE_F32, path: int = 0) -> Problem:
    return Problem(tokens, dim, hidden, n_experts, top_k, out_dtype, path)


def capacity_rows(p: Problem) -> int:
    return int(lib.moe_capacity_rows(ctypes.byref(p)))


def workspace_bytes(p: Problem) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(p)))


def decode_max_tokens() -> int:
    return int(lib.moe_decode_max_tokens())


# ---------------------------------------------------------------------------
# tensor marshalling (PyTorch supplies device memory and the stream only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, shape=None, name="tensor", optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bf16():
    torch = _torch()
    return (torch.bfloat16, torch.uint16, torch.int16)


def _shape_of(x, w1, top_k, out_dtype=MOE_F32, path=PATH_AUTO) -> Problem:
    T, D = x.shape
    n, D2, H = w1.shape
    if D2 != D:
        raise ValueError(f"w1 has dim {D2}, x has dim {D}")
    return problem(T, D, H, n, top_k, out_dtype, path)


def route_workspace_bytes(p: Problem) -> int:
    return int(lib.moe_route_workspace_bytes(ctypes.byref(p)))


def route(x, w_gate, top_k: int, topk_idx=None, topk_gate=None, logits=None, workspace=None,
          stream=None):
    """moe_route: returns (topk_idx int32 [T][K], topk_gate fp32 [T][K]).  The
    scratch the slice-wise matrix-core router needs (more than 16 experts,
    or at least 2048 tokens with a multiple of 4 experts and W_g over 64 KiB)
    is taken from `workspace` or allocated here."""
    torch = _torch()
    T, D = x.shape
    n = w_gate.shape[1]
    p = problem(T, D, 8, n, top_k)
    if topk_idx is None:
        topk_idx = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    if topk_gate is None:
        topk_gate = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    need = route_workspace_bytes(p)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = _ptr(workspace, torch.uint8, None, "workspace", optional=True)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("moe_route", lib.moe_route(
        ctypes.byref(p), _ptr(x, _bf16(), (T, D), "x"), _ptr(w_gate, _bf16(), (D, n), "w_gate"),
        _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"),
        _ptr(topk_gate, torch.float32, (T, top_k), "topk_gate"),
        _ptr(logits, torch.float32, (T, n), "logits", optional=True), ws_ptr, ws_bytes,
        _stream(stream)))
    return topk_idx, topk_gate


def permute(topk_idx, n_experts: int, stream=None, out=None):
    """moe_permute: returns dict(expert_count, expert_offset, row_slot, slot_row)."""
    torch = _torch()
    T, K = topk_idx.shape
    p = problem(T, 8, 8, n_experts, K)
    cap = capacity_rows(p)
    dev = topk_idx.device
    o = out or {}
    count = o.get("expert_count") if o.get("expert_count") is not None else torch.empty(n_experts, dtype=torch.int32, device=dev)
    offset = o.get("expert_offset") if o.get("expert_offset") is not None else torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    row_slot = o.get("row_slot") if o.get("row_slot") is not None else torch.empty(cap, dtype=torch.int32, device=dev)
    slot_row = o.get("slot_row") if o.get("slot_row") is not None else torch.empty(T * K, dtype=torch.int32, device=dev)
    _check("moe_permute", lib.moe_permute(
        ctypes.byref(p), _ptr(topk_idx, torch.int32, (T, K), "topk_idx"),
        _ptr(count, torch.int32, (n_experts,), "expert_count"),
        _ptr(offset, torch.int32, (n_experts + 1,), "expert_offset"),
        _ptr(row_slot, torch.int32, (cap,), "row_slot"),
        _ptr(slot_row, torch.int32, (T * K,), "slot_row"), _stream(stream)))
    return dict(expert_count=count, expert_offset=offset, row_slot=row_slot, slot_row=slot_row)


def grouped_ffn(x, expert_count, expert_offset, row_slot, w1, w3, w2, top_k: int,
                y_rows=None, workspace=None, stream=None, path: int = PATH_AUTO):
    """moe_grouped_ffn: returns y_rows fp32 [cap][D]."""
    torch = _torch()
    p = _shape_of(x, w1, top_k, MOE_F32, path)
    T, D, H, n = p.tokens, p.dim, p.hidden, p.n_experts
    cap = capacity_rows(p)
    if y_rows is None:
        y_rows = torch.empty((cap, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(p), dtype=torch.uint8, device=x.device)
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(
        ctypes.byref(p), _ptr(x, _bf16(), (T, D), "x"),
        _ptr(expert_count, torch.int32, (n,), "expert_count"),
        _ptr(expert_offset, torch.int32, (n + 1,), "expert_offset"),
        _ptr(row_slot, torch.int32, (cap,), "row_slot"),
        _ptr(w1, _bf16(), (n, D, H), "w1"), _ptr(w3, _bf16(), (n, D, H), "w3"),
        _ptr(w2, _bf16(), (n, H, D), "w2"), _ptr(y_rows, torch.float32, (cap, D), "y_rows"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream)))
    return y_rows


def combine(y_rows, slot_row, topk_gate, out_dtype: int = MOE_F32, out=None, stream=None):
    """moe_combine: returns out [T][D] (fp32, or bf16 when out_dtype == MOE_BF16)."""
    torch = _torch()
    T, K = topk_gate.shape
    cap, D = y_rows.shape
    p = problem(T, D, 8, max(K, 1), K, out_dtype)
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                          device=y_rows.device)
    _check("moe_combine", lib.moe_combine(
        ctypes.byref(p), _ptr(y_rows, torch.float32, None, "y_rows"),
        _ptr(slot_row, torch.int32, (T * K,), "slot_row"),
        _ptr(topk_gate, torch.float32, (T, K), "topk_gate"),
        _ptr(out, (torch.float32,) if out_dtype == MOE_F32 else _bf16(), (T, D), "out"),
        _stream(stream)))
    return out


def route_stats(topk_idx, n_experts: int, counts=None, stream=None):
    """moe_route_stats: routing diagnostics of a [T][K] expert choice tensor.

    Returns a dict of host ints / lists: ``first`` (slots per expert among
    first choices), ``any`` (slots per expert over all choices),
    ``repeat_first`` and ``repeat_either`` (consecutive-token counts), and
    ``counts`` (the raw int32 device tensor [2n+2])."""
    torch = _torch()
    T, K = topk_idx.shape
    n = int(n_experts)
    p = problem(T, 8, 8, n, K)
    if counts is None:
        counts = torch.empty(2 * n + 2, dtype=torch.int32, device=topk_idx.device)
    _check("moe_route_stats", lib.moe_route_stats(
        ctypes.byref(p), _ptr(topk_idx, torch.int32, (T, K), "topk_idx") if T else None,
        _ptr(counts, torch.int32, (2 * n + 2,), "counts"), _stream(stream)))
    c = counts.cpu().tolist()
    return {"first": c[:n], "any": c[n:2 * n], "repeat_first": c[2 * n],
            "repeat_either": c[2 * n + 1], "counts": counts}


def forward(x, w_gate, w1, w3, w2, top_k: int, out=None, topk_idx=None, topk_gate=None,
            workspace=None, out_dtype: int = MOE_F32, stream=None, events=None,
            path: int = PATH_AUTO):
    """moe_forward: the whole layer.  Returns out [T][D].

    ``events``: optional sequence of 6 raw hipEvent_t handles (None entries
    are skipped); then moe_forward_timed records them between the stages.  ``path``: PATH_AUTO,
    PATH_STREAM (weight streaming, T <= STREAM_MAX_TOKENS) or PATH_TILED."""
    torch = _torch()
    p = _shape_of(x, w1, top_k, out_dtype, path)
    T, D, H, n = p.tokens, p.dim, p.hidden, p.n_experts
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32,
                          device=x.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(p), dtype=torch.uint8, device=x.device)
    args = (ctypes.byref(p), _ptr(x, _bf16(), (T, D), "x"), _ptr(w_gate, _bf16(), (D, n), "w_gate"),
            _ptr(w1, _bf16(), (n, D, H), "w1"), _ptr(w3, _bf16(), (n, D, H), "w3"),
            _ptr(w2, _bf16(), (n, H, D), "w2"),
            _ptr(out, (torch.float32,) if out_dtype == MOE_F32 else _bf16(), (T, D), "out"),
            _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx", optional=True),
            _ptr(topk_gate, torch.float32, (T, top_k), "topk_gate", optional=True),
            _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    if events is None:
        _check("moe_forward", lib.moe_forward(*args))
    else:
        if len(events) != 6:
            raise ValueError("events must hold 6 hipEvent_t handles")
        arr = (_vp * 6)(*events)
        _check("moe_forward_timed", lib.moe_forward_timed(*args, arr))
    return out


def forward_noalloc(x, w_gate, w1, w3, w2, top_k: int, out, topk_idx=None, topk_gate=None,
                    out_dtype: int = MOE_F32, stream=None, path: int = PATH_AUTO):
    """moe_forward_noalloc: the whole layer with no workspace (the library's
    own device array holds the intermediates).  For the batches moe_forward
    streams; `out` (and the optional routing outputs) must be given, since
    this call is for callers that do not allocate.  Returns out."""
    torch = _torch()
    p = _shape_of(x, w1, top_k, out_dtype, path)
    T, D, H, n = p.tokens, p.dim, p.hidden, p.n_experts
    _check("moe_forward_noalloc", lib.moe_forward_noalloc(
        ctypes.byref(p), _ptr(x, _bf16(), (T, D), "x"), _ptr(w_gate, _bf16(), (D, n), "w_gate"),
        _ptr(w1, _bf16(), (n, D, H), "w1"), _ptr(w3, _bf16(), (n, D, H), "w3"),
        _ptr(w2, _bf16(), (n, H, D), "w2"),
        _ptr(out, (torch.float32,) if out_dtype == MOE_F32 else _bf16(), (T, D), "out"),
        _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx", optional=True),
        _ptr(topk_gate, torch.float32, (T, top_k), "topk_gate", optional=True),
        _stream(stream)))
    return out
