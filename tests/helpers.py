"""Shared test helpers: move seeded bf16 storage buffers to the GPU and read
results back as float64.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np


def to_device(buf: np.ndarray, shape, strides, device="cuda"):
    """A bf16 tensor viewing `buf` (uint16 bf16 patterns) with element strides."""
    import torch
    flat = torch.from_numpy(np.ascontiguousarray(buf).view(np.int16)).to(device).view(torch.bfloat16)
    return flat.as_strided(tuple(shape), tuple(strides))


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gemm_operands(case, device="cuda"):
    A = to_device(case.A, (case.M, case.K), (case.sam, case.sak), device)
    B = to_device(case.B, (case.K, case.N), (case.sbk, case.sbn), device)
    return A, B


def sample_indices(M, N, n, seed, tile=256):
    """n random entries plus the corners and the last row/column of each ragged tail."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n))
    cols = list(rng.integers(0, N, n))
    for i in (0, M - 1):
        for j in (0, N - 1):
            rows.append(i)
            cols.append(j)
    lastr = np.arange(max(0, (M - 1) // tile * tile), M)
    lastc = np.arange(max(0, (N - 1) // tile * tile), N)
    for i in lastr[:: max(1, len(lastr) // 16)]:
        rows.append(int(i))
        cols.append(int(rng.integers(0, N)))
    for j in lastc[:: max(1, len(lastc) // 16)]:
        rows.append(int(rng.integers(0, M)))
        cols.append(int(j))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)
