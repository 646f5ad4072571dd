"""Shared test helpers (sampling of output entries); device movement comes from
synth.device.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np

from synth.device import gemm_operands, lincomp_operands, ragged_operands, to_device, to_f64  # noqa: F401


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
