"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only draws random numbers and rounds them to bf16 storage; it holds
none of the method's arithmetic.  Both sides receive the same uint16 bf16 bit
patterns, so a value can never differ between what the oracle and the GPU see.

Recipe (stable; every stored expected value depends on it):

* A tensor is a flat buffer in its storage order.  It is cut into chunks of
  ``CHUNK`` elements; chunk ``i`` of tensor ``t`` of workload seed ``s`` and
  sub-workload ``sub`` is drawn from
  ``Generator(PCG64(SeedSequence(s, spawn_key=(sub, t, i))))``.  The result is
  independent of how many threads fill the chunks.
* ``uniform``: fp32 ``u*(hi-lo)+lo`` with ``u`` from ``Generator.random`` on
  [0,1); ``normal``: fp32 ``std * standard_normal``; ``int``: integers in
  [lo, hi] converted exactly.
* fp32 samples become bf16 by IEEE round-to-nearest-even on the bit pattern:
  ``(x + 0x7FFF + ((x >> 16) & 1)) >> 16``.  NaN cannot occur with these
  distributions.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE binary16 (numpy's conversion: round to nearest,
    ties to even); returns uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _draw_chunk(seed: int, key: tuple, n: int, dist: str, p0: float, p1: float, fmt: str = "bf16") -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))
    if dist == "uniform":
        x = rng.random(n, dtype=np.float32)
        x *= np.float32(p1 - p0)
        x += np.float32(p0)
    elif dist == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(p1)
    elif dist == "int":
        x = rng.integers(int(p0), int(p1) + 1, size=n).astype(np.float32)
    else:
        raise ValueError(dist)
    return f32_to_f16_rne(x) if fmt == "f16" else f32_to_bf16_rne(x)


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def bf16_tensor(numel: int, dist: str, p0: float, p1: float, *, seed: int, sub: int = 0,
                tensor: int = 0, fmt: str = "bf16") -> np.ndarray:
    """Flat uint16 buffer of ``numel`` bf16 values drawn per the module recipe.

    ``dist``/``p0``/``p1``: ("uniform", lo, hi), ("normal", mean-ignored, std) or
    ("int", lo, hi).
    """
    out = np.empty(numel, dtype=np.uint16)
    nchunks = (numel + CHUNK - 1) // CHUNK

    def work(i: int) -> None:
        lo = i * CHUNK
        hi = min(numel, lo + CHUNK)
        out[lo:hi] = _draw_chunk(seed, (sub, tensor, i), hi - lo, dist, p0, p1, fmt)

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


# ---------------------------------------------------------------------------
# Workloads.  Each returns plain numpy uint16 storage buffers plus the element
# strides that describe them; nothing here is on a device.
# ---------------------------------------------------------------------------

class GemmCase:
    """C = A.B with A[i,k] = A_buf[i*sam + k*sak], B[k,j] = B_buf[k*sbk + j*sbn]."""

    def __init__(self, name, M, N, K, A, sam, sak, B, sbk, sbn, out_dtype, in_dtype="bf16"):
        self.name, self.M, self.N, self.K = name, M, N, K
        self.A, self.sam, self.sak = A, sam, sak
        self.B, self.sbk, self.sbn = B, sbk, sbn
        self.out_dtype = out_dtype  # "f32", "bf16" or "f16"
        self.in_dtype = in_dtype    # format of A and B: "bf16" or "f16"

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def gemm_case(M, N, K, *, dist=("uniform", -1.0, 1.0), b_dist=None, seed=0, sub=0, a_col_major=False,
              b_col_major=False, lda=None, ldb=None, out_dtype="f32", in_dtype="bf16", name="gemm") -> GemmCase:
    """A row-major [M][lda>=K] or column-major [K][lda>=M]; B row-major
    [K][ldb>=N] or column-major [N][ldb>=K]; A and B in ``in_dtype`` ("bf16"
    or "f16")."""
    b_dist = b_dist or dist
    if a_col_major:
        lda = M if lda is None else lda
        A = bf16_tensor(K * lda, *dist, seed=seed, sub=sub, tensor=0, fmt=in_dtype)
        sam, sak = 1, lda
    else:
        lda = K if lda is None else lda
        A = bf16_tensor(M * lda, *dist, seed=seed, sub=sub, tensor=0, fmt=in_dtype)
        sam, sak = lda, 1
    if b_col_major:
        ldb = K if ldb is None else ldb
        B = bf16_tensor(N * ldb, *b_dist, seed=seed, sub=sub, tensor=1, fmt=in_dtype)
        sbk, sbn = 1, ldb
    else:
        ldb = N if ldb is None else ldb
        B = bf16_tensor(K * ldb, *b_dist, seed=seed, sub=sub, tensor=1, fmt=in_dtype)
        sbk, sbn = ldb, 1
    return GemmCase(name, M, N, K, A, sam, sak, B, sbk, sbn, out_dtype, in_dtype)


GEMM_WORKLOADS = {
    # name: (M, N, K, kwargs)
    "gemm_256": (256, 256, 256, dict(dist=("uniform", -1.0, 1.0), seed=1, out_dtype="f32")),
    "gemm_4096": (4096, 4096, 4096, dict(dist=("normal", 0.0, 1.0), seed=2, out_dtype="bf16")),
    "ffn_up": (16384, 28672, 8192, dict(dist=("normal", 0.0, 1.0), b_dist=("normal", 0.0, 0.02),
                                        seed=3, sub=0, out_dtype="bf16")),
    "ffn_down": (16384, 8192, 28672, dict(dist=("normal", 0.0, 1.0), b_dist=("normal", 0.0, 0.02),
                                          seed=3, sub=1, out_dtype="bf16")),
    "edge": (8191, 5003, 4099, dict(dist=("uniform", -1.0, 1.0), seed=5, sub=0, b_col_major=True,
                                    out_dtype="f32")),
    "skinny_splitk": (128, 8192, 65536, dict(dist=("uniform", -1.0, 1.0), seed=5, sub=1,
                                             out_dtype="f32")),
    # mid-size: 288 tiles of 256x128 leave a second pass 1/8 full; the plan's
    # tile-count rule takes 192 tiles of 192x256 in one pass instead
    "gemm_3000": (3000, 3000, 3000, dict(dist=("normal", 0.0, 1.0), seed=11, out_dtype="bf16")),
    # fp16 operands and output (the pages' GEMM tables are fp16)
    "gemm_4096_f16": (4096, 4096, 4096, dict(dist=("normal", 0.0, 1.0), seed=7, out_dtype="f16",
                                             in_dtype="f16")),
    # C = X W^T with W stored [N][K]: B K-contiguous (a linear layer's usual weight layout)
    "gemm_4096_nt": (4096, 4096, 4096, dict(dist=("normal", 0.0, 1.0), seed=2, out_dtype="bf16", b_col_major=True)),
    # C = X^T Y: A M-contiguous (a layer's weight gradient dW = dY^T X)
    "gemm_4096_tn": (4096, 4096, 4096, dict(dist=("normal", 0.0, 1.0), seed=2, out_dtype="bf16", a_col_major=True)),
}


def gemm_workload(name: str) -> GemmCase:
    M, N, K, kw = GEMM_WORKLOADS[name]
    return gemm_case(M, N, K, name=name, **kw)


class LincompCase:
    """Per candidate (r, c): X = [user[r]; item[r, c]] of shape [(Nu+Ni), D];
    Y[r, c] = W^T . X of shape [Mo, D].  All buffers dense, last dim contiguous."""

    def __init__(self, name, R, C, Nu, Ni, D, Mo, user, item, W):
        self.name, self.R, self.C, self.Nu, self.Ni, self.D, self.Mo = name, R, C, Nu, Ni, D, Mo
        self.user, self.item, self.W = user, item, W

    @property
    def strides(self):
        return dict(su_r=self.Nu * self.D, su_n=self.D,
                    si_r=self.C * self.Ni * self.D, si_c=self.Ni * self.D, si_n=self.D,
                    sw_n=self.Mo,
                    sy_r=self.C * self.Mo * self.D, sy_c=self.Mo * self.D, sy_m=self.D)

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the deduplicated layer must move: user and item once, W once, Y once (bf16)."""
        return 2 * (self.R * self.Nu * self.D + self.R * self.C * self.Ni * self.D
                    + (self.Nu + self.Ni) * self.Mo + self.R * self.C * self.Mo * self.D)

    @property
    def flops(self) -> float:
        return 2.0 * self.Mo * self.D * (self.R * self.Nu + self.R * self.C * self.Ni)


def lincomp_case(R, C, Nu=256, Ni=256, D=256, Mo=64, *, x_dist=("normal", 0.0, 0.1),
                 w_dist=("normal", 0.0, 0.05), seed=4, sub=0, name="lincomp") -> LincompCase:
    user = bf16_tensor(R * Nu * D, *x_dist, seed=seed, sub=sub, tensor=0)
    item = bf16_tensor(R * C * Ni * D, *x_dist, seed=seed, sub=sub, tensor=1)
    W = bf16_tensor((Nu + Ni) * Mo, *w_dist, seed=seed, sub=sub, tensor=2)
    return LincompCase(name, R, C, Nu, Ni, D, Mo, user, item, W)


def lincomp_workload(name: str = "lincomp_256x128") -> LincompCase:
    if name == "lincomp_256x128":
        return lincomp_case(256, 128, name=name)
    if name == "lincomp_small":
        return lincomp_case(3, 5, name=name, sub=1)
    raise KeyError(name)


class RaggedLincompCase:
    """Ragged requests: request r owns candidates offsets[r] .. offsets[r+1]-1
    of a flat candidate axis.  user [R][Nu][D], item [Ctot][Ni][D],
    W [Nu+Ni][Mo], Y [Ctot][Mo][D]; dense, last dim contiguous."""

    def __init__(self, name, lengths, Nu, Ni, D, Mo, user, item, W):
        self.name, self.Nu, self.Ni, self.D, self.Mo = name, Nu, Ni, D, Mo
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.R = int(self.lengths.shape[0])
        self.offsets = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)
        self.Ctot = int(self.offsets[-1])
        self.user, self.item, self.W = user, item, W

    def request_of(self, g: int) -> int:
        """The request owning flat candidate g."""
        return int(np.searchsorted(self.offsets, g, side="right") - 1)

    @property
    def dims(self):
        """(R, C, Nu, Ni, D, Mo) for the per-candidate oracle, C = Ctot."""
        return (self.R, self.Ctot, self.Nu, self.Ni, self.D, self.Mo)

    @property
    def strides(self):
        """Element strides; the flat candidate axis has no request stride."""
        return dict(su_r=self.Nu * self.D, su_n=self.D, si_r=0, si_c=self.Ni * self.D, si_n=self.D,
                    sw_n=self.Mo, sy_c=self.Mo * self.D, sy_m=self.D)

    @property
    def algorithmic_bytes(self) -> int:
        """user once per request, every item row once, W once, Y once (bf16)."""
        return 2 * (self.R * self.Nu * self.D + self.Ctot * self.Ni * self.D
                    + (self.Nu + self.Ni) * self.Mo + self.Ctot * self.Mo * self.D)


def ragged_lengths(R: int, median: float, sigma: float, *, seed: int, sub: int = 0, lo: int = 1,
                   hi: int = 1024) -> np.ndarray:
    """Candidates per request: round(median * exp(sigma * z)), z standard
    normal (a lognormal length mix), clipped to [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(sub, 99, 0))))
    z = rng.standard_normal(R)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)


def lincomp_ragged_case(lengths, Nu=256, Ni=256, D=256, Mo=64, *, x_dist=("normal", 0.0, 0.1),
                        w_dist=("normal", 0.0, 0.05), seed=6, sub=0, name="lincomp_ragged") -> RaggedLincompCase:
    lengths = np.asarray(lengths, dtype=np.int64)
    R, Ctot = int(lengths.shape[0]), int(lengths.sum())
    user = bf16_tensor(R * Nu * D, *x_dist, seed=seed, sub=sub, tensor=0)
    item = bf16_tensor(Ctot * Ni * D, *x_dist, seed=seed, sub=sub, tensor=1)
    W = bf16_tensor((Nu + Ni) * Mo, *w_dist, seed=seed, sub=sub, tensor=2)
    return RaggedLincompCase(name, lengths, Nu, Ni, D, Mo, user, item, W)


def lincomp_ragged_workload(name: str = "lincomp_ragged_256") -> RaggedLincompCase:
    """256 requests, lognormal candidate counts (median 112, sigma 0.5: mean
    about 127, so the total is close to the 256 x 128 workload)."""
    if name == "lincomp_ragged_256":
        return lincomp_ragged_case(ragged_lengths(256, 112.0, 0.5, seed=6), seed=6, name=name)
    raise KeyError(name)
