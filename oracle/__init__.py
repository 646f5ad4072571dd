"""fp64 CPU oracle (ctypes wrapper over oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path; both receive the same bf16 bit patterns from the ``synth`` module.

Every function takes flat numpy uint16 storage buffers plus element strides
and returns float64 arrays.  See oracle.h for the definitions.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_get_threads.restype = ctypes.c_int
        lib.oracle_gemm_rows.argtypes = [_i64] * 3 + [_p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p, _p]
        lib.oracle_gemm_entries.argtypes = [_i64] * 3 + [_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _p, _p, _p]
        lib.oracle_gemm_rows_fmt.argtypes = [ctypes.c_int] + lib.oracle_gemm_rows.argtypes
        lib.oracle_gemm_entries_fmt.argtypes = [ctypes.c_int] + lib.oracle_gemm_entries.argtypes
        lib.oracle_widen.argtypes = [ctypes.c_int, _i64, _p, _p]
        lib.oracle_epilogue.argtypes = [ctypes.c_int, _i64, _i64, _p, _p, _p]
        lc = [_i64] * 6 + [_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _i64, _p, _p, _p]
        lib.oracle_lincomp_naive.argtypes = lc + [_p]
        lib.oracle_lincomp_dedup.argtypes = lc
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are 16-bit bit patterns (uint16)")
    return a.reshape(-1)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


FORMATS = {"bf16": 0, "f16": 2}  # element formats of the 16-bit inputs


def widen(bits, fmt="bf16") -> np.ndarray:
    """Exact fp64 values of 16-bit patterns in format ``fmt``."""
    bits = _u16(bits)
    out = np.empty(bits.shape[0], dtype=np.float64)
    _load().oracle_widen(FORMATS[fmt], bits.shape[0], _ptr(bits), _ptr(out))
    return out


def gemm(M, N, K, A, sam, sak, B, sbk, sbn, *, rows=None, bound=True, fmt="bf16"):
    """Rows ``rows=(row0, nrows)`` (default: all) of C = A.B and of S = sum |a*b|;
    A and B hold ``fmt`` ("bf16" or "f16") bit patterns."""
    lib = _load()
    A, B = _u16(A), _u16(B)
    row0, nrows = (0, M) if rows is None else rows
    C = np.empty((nrows, N), dtype=np.float64)
    S = np.empty((nrows, N), dtype=np.float64) if bound else None
    lib.oracle_gemm_rows_fmt(FORMATS[fmt], M, N, K, _ptr(A), sam, sak, _ptr(B), sbk, sbn, row0, nrows,
                             _ptr(C), _ptr(S) if bound else None)
    return (C, S) if bound else C


def gemm_entries(M, N, K, A, sam, sak, B, sbk, sbn, rows, cols, fmt="bf16"):
    """C[rows[e], cols[e]] and S at the same entries."""
    lib = _load()
    A, B = _u16(A), _u16(B)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    S = np.empty(rows.shape[0], dtype=np.float64)
    lib.oracle_gemm_entries_fmt(FORMATS[fmt], M, N, K, _ptr(A), sam, sak, _ptr(B), sbk, sbn, rows.shape[0],
                            _ptr(rows), _ptr(cols), _ptr(out), _ptr(S))
    return out, S


def _lc_args(case_dims, user, item, W, strides, pairs):
    R, C, Nu, Ni, D, Mo = case_dims
    rr = np.ascontiguousarray([p[0] for p in pairs], dtype=np.int64)
    cc = np.ascontiguousarray([p[1] for p in pairs], dtype=np.int64)
    for r, c in pairs:
        if not (0 <= r < R and 0 <= c < C):
            raise IndexError((r, c))
    s = strides
    return rr, cc, [R, C, Nu, Ni, D, Mo, _ptr(user), s["su_r"], s["su_n"], _ptr(item), s["si_r"],
                    s["si_c"], s["si_n"], _ptr(W), s["sw_n"], len(pairs), _ptr(rr), _ptr(cc)]


def lincomp_naive(dims, user, item, W, strides, pairs, *, bound=True):
    """Y[p] (and S[p]) for candidates pairs[p] = (r, c), computed per candidate
    from the stacked input X = [user[r]; item[r, c]]."""
    lib = _load()
    user, item, W = _u16(user), _u16(item), _u16(W)
    Mo, D = dims[5], dims[4]
    rr, cc, args = _lc_args(dims, user, item, W, strides, pairs)
    Y = np.empty((len(pairs), Mo, D), dtype=np.float64)
    S = np.empty((len(pairs), Mo, D), dtype=np.float64) if bound else None
    lib.oracle_lincomp_naive(*args, _ptr(Y), _ptr(S) if bound else None)
    return (Y, S) if bound else Y


def lincomp_dedup(dims, user, item, W, strides, pairs):
    """Y[p] by the user-once rewrite (U + V); used to check the rewrite's invariance."""
    lib = _load()
    user, item, W = _u16(user), _u16(item), _u16(W)
    Mo, D = dims[5], dims[4]
    rr, cc, args = _lc_args(dims, user, item, W, strides, pairs)
    Y = np.empty((len(pairs), Mo, D), dtype=np.float64)
    lib.oracle_lincomp_dedup(*args, _ptr(Y))
    return Y


def lincomp_case(case, pairs, *, bound=True, naive=True):
    dims = (case.R, case.C, case.Nu, case.Ni, case.D, case.Mo)
    if naive:
        return lincomp_naive(dims, case.user, case.item, case.W, case.strides, pairs, bound=bound)
    return lincomp_dedup(dims, case.user, case.item, case.W, case.strides, pairs)


def gemm_case(case, *, rows=None, bound=True):
    return gemm(case.M, case.N, case.K, case.A, case.sam, case.sak, case.B, case.sbk, case.sbn,
                rows=rows, bound=bound, fmt=case.in_dtype)


def gemm_case_entries(case, rows, cols):
    return gemm_entries(case.M, case.N, case.K, case.A, case.sam, case.sak, case.B, case.sbk,
                        case.sbn, rows, cols, fmt=case.in_dtype)


ACTS = {None: 0, "relu": 1, "gelu": 2, "silu": 3}


def epilogue(C, S, bias, act, cols=None):
    """act(C + bias) in fp64 and S + |bias| (new arrays).  C, S: [rows][N], or
    1-D values at columns ``cols`` (sampled entries); bias: fp32 [N] or None."""
    lib = _load()
    C = np.array(C, dtype=np.float64, copy=True)
    S = np.array(S, dtype=np.float64, copy=True) if S is not None else None
    if cols is not None:
        b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32)[np.asarray(cols)])
        for k in range(C.shape[0]):
            bk = None if b is None else b[k:k + 1]
            ck = C[k:k + 1]
            sk = S[k:k + 1] if S is not None else None
            lib.oracle_epilogue(ACTS[act], 1, 1, _ptr(ck), _ptr(sk) if sk is not None else None,
                                _ptr(bk) if bk is not None else None)
            C[k] = ck[0]
            if S is not None:
                S[k] = sk[0]
        return C, S
    C = np.ascontiguousarray(C)
    rows, N = C.shape
    b = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float32))
    lib.oracle_epilogue(ACTS[act], rows, N, _ptr(C), _ptr(S) if S is not None else None,
                        _ptr(b) if b is not None else None)
    return C, S


def lincomp_epilogue(Y, S, bias, act):
    """The fused epilogue of linear compression in fp64: act(Y[p][m][d] +
    bias[m]) for every candidate p, with S[p][m][d] + |bias[m]| (page "Meta
    accélère un noyau GPU d'un facteur 4 avec TLX", section "Par où commencer
    dans votre équipe": fuse steps, then measure again).  The bias is one
    value per compressed row m, so each candidate's [Mo][D] block is seen as
    [D][Mo] (rows d, columns m) by the GEMM epilogue above, whose bias runs
    along columns; the arithmetic is that function's.  Y, S: [P][Mo][D];
    bias: fp32 [Mo] or None; S may be None."""
    Y = np.asarray(Y, dtype=np.float64)
    P, Mo, D = Y.shape
    Yt = np.ascontiguousarray(Y.transpose(0, 2, 1)).reshape(P * D, Mo)
    St = None if S is None else np.ascontiguousarray(np.asarray(S, dtype=np.float64).transpose(0, 2, 1)).reshape(
        P * D, Mo)
    Yo, So = epilogue(Yt, St, bias, act)
    Yo = Yo.reshape(P, D, Mo).transpose(0, 2, 1)
    So = None if So is None else So.reshape(P, D, Mo).transpose(0, 2, 1)
    return np.ascontiguousarray(Yo), (None if So is None else np.ascontiguousarray(So))

