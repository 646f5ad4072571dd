"""Per-element acceptance bound for a GPU result against the fp64 oracle.

TEST INFRASTRUCTURE ONLY.  For an output element with oracle value ``ref`` and
``S = sum |a*b|`` over the same terms:

* fp32 output: ``|gpu - ref| <= 1e-3 * S + 1e-6``
* bf16 output: the same plus ``2**-8 * |ref|``; this extra term is the
  half-unit-in-the-last-place of an 8-significant-bit bf16 value, i.e. the
  largest error of a round-to-nearest-even conversion.  A truncating
  conversion can err by almost a whole unit and therefore fails it.
* fp16 output: the fp32 bound plus ``2**-11 * |ref|``, the half unit of an
  11-significant-bit fp16 value (normal range; below it the absolute 1e-6
  covers the subnormal half unit 2**-25).
"""
from __future__ import annotations

import numpy as np


# Largest |slope| of each activation (ReLU 1; GELU max of Phi(x) + x phi(x)
# = 1.1289 at x = sqrt 2; SiLU 1.0998): an error e in the sum moves the
# activated value by at most L * e.
ACT_SLOPE = {None: 1.0, "relu": 1.0, "gelu": 1.13, "silu": 1.10}


def bound(ref: np.ndarray, S: np.ndarray, out_dtype: str, act=None) -> np.ndarray:
    """With an activation: S is the sum of |terms| including |bias|; the fp32
    sum's bound is scaled by the activation's slope, and 5e-7 * S covers the
    fp32 evaluation of the activation (its argument is at most S)."""
    S = np.asarray(S, dtype=np.float64)
    b = ACT_SLOPE[act] * (1e-3 * S + 1e-6)
    if act in ("gelu", "silu"):
        b = b + 5e-7 * S
    if out_dtype == "bf16":
        b = b + 2.0 ** -8 * np.abs(np.asarray(ref, dtype=np.float64))
    elif out_dtype == "f16":
        b = b + 2.0 ** -11 * np.abs(np.asarray(ref, dtype=np.float64))
    elif out_dtype != "f32":
        raise ValueError(out_dtype)
    return b


def check(gpu, ref, S, out_dtype: str, act=None):
    """Returns (ok, worst_ratio, worst_flat_index); ratio = |err| / bound (ok iff <= 1,
    and no NaN/Inf in gpu)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.shape != ref.shape:
        raise ValueError(f"shape mismatch {gpu.shape} vs {ref.shape}")
    if gpu.size == 0:
        return True, 0.0, -1
    if not np.all(np.isfinite(gpu)):
        idx = int(np.flatnonzero(~np.isfinite(gpu.reshape(-1)))[0])
        return False, float("inf"), idx
    ratio = np.abs(gpu - ref) / bound(ref, S, out_dtype, act)
    idx = int(np.argmax(ratio))
    worst = float(ratio.reshape(-1)[idx])
    return worst <= 1.0, worst, idx


def assert_close(gpu, ref, S, out_dtype: str, what: str = "", act=None) -> float:
    ok, worst, idx = check(gpu, ref, S, out_dtype, act)
    if not ok:
        g = np.asarray(gpu, dtype=np.float64).reshape(-1)
        r = np.asarray(ref, dtype=np.float64).reshape(-1)
        s = np.asarray(S, dtype=np.float64).reshape(-1)
        raise AssertionError(
            f"{what}: element {idx} outside tolerance: gpu={g[idx]!r} ref={r[idx]!r} "
            f"S={s[idx]!r} err/bound={worst:.3g}")
    return worst
