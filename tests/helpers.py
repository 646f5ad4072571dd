"""Shared test helpers (sampling of output entries); device movement comes from
synth.device.  No arithmetic of the method lives here."""
from __future__ import annotations

import re

import numpy as np

from synth.device import gemm_operands, lincomp_operands, ragged_operands, to_device, to_f64  # noqa: F401


def sample_indices(M, N, n, seed, tile=256):
    """n random entries plus the corners and the last row/column of each ragged
    tail.  tile: the output tile, an int or (rows, cols)."""
    tm, tn = (tile, tile) if isinstance(tile, int) else tile
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, n))
    cols = list(rng.integers(0, N, n))
    for i in (0, M - 1):
        for j in (0, N - 1):
            rows.append(i)
            cols.append(j)
    lastr = np.arange(max(0, (M - 1) // tm * tm), M)
    lastc = np.arange(max(0, (N - 1) // tn * tn), N)
    for i in lastr[:: max(1, len(lastr) // 16)]:
        rows.append(int(i))
        cols.append(int(rng.integers(0, N)))
    for j in lastc[:: max(1, len(lastc) // 16)]:
        rows.append(int(rng.integers(0, M)))
        cols.append(int(j))
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def plan_tile(describe: str) -> tuple[int, int]:
    """The output tile (rows, cols) a plan description names ("tile=256x256")."""
    m = re.search(r"\btile=(\d+)x(\d+)", describe)
    if not m:
        raise ValueError(f"no tile in plan description: {describe}")
    return int(m.group(1)), int(m.group(2))


def per_tile_indices(M, N, tile, seed):
    """One seeded random entry inside every output tile of the (rows, cols)
    tile grid that covers M x N (clipped at the ragged edges)."""
    tm, tn = tile
    rng = np.random.default_rng(seed)
    gm, gn = -(-M // tm), -(-N // tn)
    ti, tj = np.meshgrid(np.arange(gm), np.arange(gn), indexing="ij")
    r0, c0 = ti.ravel() * tm, tj.ravel() * tn
    hr = np.minimum(r0 + tm, M) - r0
    hc = np.minimum(c0 + tn, N) - c0
    rows = r0 + (rng.random(r0.shape[0]) * hr).astype(np.int64)
    cols = c0 + (rng.random(c0.shape[0]) * hc).astype(np.int64)
    return rows.astype(np.int64), cols.astype(np.int64)


def strip_starts(M, nrows, seed):
    """Row strips checked in full at large sizes: a seeded strip of nrows rows,
    plus the first and the last row (as (start, count) pairs)."""
    rng = np.random.default_rng(seed)
    start = int(rng.integers(0, max(1, M - nrows + 1)))
    out = [(start, min(nrows, M - start)), (0, 1), (M - 1, 1)]
    return out
