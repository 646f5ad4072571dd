"""Move seeded bf16 storage buffers to the GPU and read results back.
Data movement only: no arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np


def to_device(buf: np.ndarray, shape, strides, device="cuda", fmt="bf16"):
    """A bf16 (or fmt "f16": fp16) tensor viewing `buf` (uint16 patterns) with element strides."""
    import torch
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    flat = torch.from_numpy(np.ascontiguousarray(buf).view(np.int16)).to(device).view(dt)
    return flat.as_strided(tuple(shape), tuple(strides))


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gemm_operands(case, device="cuda"):
    fmt = getattr(case, "in_dtype", "bf16")
    A = to_device(case.A, (case.M, case.K), (case.sam, case.sak), device, fmt)
    B = to_device(case.B, (case.K, case.N), (case.sbk, case.sbn), device, fmt)
    return A, B


def lincomp_operands(case, device="cuda"):
    c = case
    z = np.zeros(8, np.uint16)
    user = to_device(c.user if c.Nu else z, (c.R, c.Nu, c.D), (c.Nu * c.D, c.D, 1), device)
    item = to_device(c.item if c.Ni else z, (c.R, c.C, c.Ni, c.D), (c.C * c.Ni * c.D, c.Ni * c.D, c.D, 1),
                     device)
    W = to_device(c.W, (c.Nu + c.Ni, c.Mo), (c.Mo, 1), device)
    return user, item, W


def ragged_operands(case, device="cuda"):
    """user [R][Nu][D], item [Ctot][Ni][D], W, and the int64 offsets [R+1] on the device."""
    import torch
    c = case
    z = np.zeros(8, np.uint16)
    user = to_device(c.user if c.Nu else z, (c.R, c.Nu, c.D), (c.Nu * c.D, c.D, 1), device)
    item = to_device(c.item if (c.Ni and c.Ctot) else z, (c.Ctot, c.Ni, c.D), (c.Ni * c.D, c.D, 1), device)
    W = to_device(c.W, (c.Nu + c.Ni, c.Mo), (c.Mo, 1), device)
    offsets = torch.from_numpy(c.offsets.copy()).to(device)
    return user, item, W, offsets
