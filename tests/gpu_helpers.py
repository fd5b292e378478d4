"""Shared helpers for the GPU parity tests (inputs to the device, outputs back)."""
import numpy as np


def dev_bf16(a: np.ndarray):
    """bf16 bit patterns (uint16) -> torch.bfloat16 tensor on cuda:0."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def dev_i32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def expected_permutation(idx: np.ndarray, n: int, tile_m: int, cap: int):
    """Stable grouping of slots t*K+k by expert with segments padded to tile_m:
    the index bookkeeping the permute step must reproduce exactly."""
    flat = idx.reshape(-1)
    P = flat.size
    count = np.array([(flat == e).sum() for e in range(n)], np.int32)
    padded = (count + tile_m - 1) // tile_m * tile_m
    offset = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    row_slot = np.full(cap, -1, np.int32)
    slot_row = np.full(P, -1, np.int32)
    for e in range(n):
        slots = np.nonzero(flat == e)[0]
        rows = offset[e] + np.arange(slots.size)
        row_slot[rows] = slots
        slot_row[slots] = rows
    return count, offset, row_slot, slot_row
