"""bf16 GEMM and RecSys linear-compression layer for MI355X (gfx950).

Thin Python binding over liblinlayers.so, whose C ABI is declared in
include/linlayers.h.  The functions named like the C entry points
(gemm_plan_create, gemm_run, lincomp_run, ...) only marshal arguments; every
step of the computation runs in the library's HIP kernels.  ``gemm`` and
``lincomp`` are torch conveniences over them (torch supplies device memory and
the current stream).

Importing this module fails if the library has not been built
(``python recsys_linear_layers_amd/build.py``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinlayers.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python {os.path.join(_HERE, 'build.py')}` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

LL_OK, LL_ERR_INVALID_ARG, LL_ERR_UNSUPPORTED, LL_ERR_WORKSPACE, LL_ERR_HIP, LL_ERR_NO_DEVICE = range(6)
LL_BF16, LL_F32, LL_F16 = 0, 1, 2
LL_EPI_BIAS, LL_EPI_RELU, LL_EPI_GELU, LL_EPI_SILU = 0x1, 0x10, 0x20, 0x30
ACTIVATIONS = {None: 0, "relu": LL_EPI_RELU, "gelu": LL_EPI_GELU, "silu": LL_EPI_SILU}
LL_FLAG_PACK_A = 0x1
LL_FLAG_PACK_B = 0x2
LL_FLAG_PRODUCER_CONSUMER = 0x4
LL_FLAG_COOPERATIVE = 0x8
LL_LINCOMP_NO_DEDUP = 0x1

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class GemmDesc(ctypes.Structure):
    _fields_ = [("M", _i64), ("N", _i64), ("K", _i64),
                ("stride_am", _i64), ("stride_ak", _i64), ("stride_bk", _i64), ("stride_bn", _i64),
                ("stride_cm", _i64), ("stride_cn", _i64),
                ("a_type", ctypes.c_int32), ("b_type", ctypes.c_int32), ("c_type", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("epilogue", ctypes.c_uint32)]


class LincompDesc(ctypes.Structure):
    _fields_ = [("R", _i64), ("C", _i64), ("Nu", _i64), ("Ni", _i64), ("D", _i64), ("Mo", _i64),
                ("su_r", _i64), ("su_c", _i64), ("su_n", _i64),
                ("si_r", _i64), ("si_c", _i64), ("si_n", _i64),
                ("sw_n", _i64),
                ("sy_r", _i64), ("sy_c", _i64), ("sy_m", _i64),
                ("y_type", ctypes.c_int32), ("flags", ctypes.c_uint32), ("epilogue", ctypes.c_uint32)]


class LincompRaggedDesc(ctypes.Structure):
    _fields_ = [("R", _i64), ("Ctot", _i64), ("Nu", _i64), ("Ni", _i64), ("D", _i64), ("Mo", _i64),
                ("su_r", _i64), ("su_n", _i64),
                ("si_c", _i64), ("si_n", _i64),
                ("sw_n", _i64),
                ("sy_c", _i64), ("sy_m", _i64),
                ("y_type", ctypes.c_int32), ("flags", ctypes.c_uint32), ("epilogue", ctypes.c_uint32)]


_lib.ll_status_string.restype = ctypes.c_char_p
_lib.ll_status_string.argtypes = [ctypes.c_int]
_lib.ll_last_error.restype = ctypes.c_char_p
_lib.ll_last_error.argtypes = []
_lib.gemm_plan_create.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(GemmDesc)]
_lib.gemm_plan_workspace_size.argtypes = [_vp, ctypes.POINTER(ctypes.c_size_t)]
_lib.gemm_plan_describe.argtypes = [_vp, ctypes.c_char_p, ctypes.c_size_t]
_lib.gemm_run.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.gemm_run_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.gemm_run_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
_lib.gemm_plan_destroy.argtypes = [_vp]
_lib.lincomp_workspace_size.argtypes = [ctypes.POINTER(LincompDesc), ctypes.POINTER(ctypes.c_size_t)]
_lib.lincomp_run.argtypes = [ctypes.POINTER(LincompDesc), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.lincomp_ragged_run.argtypes = [ctypes.POINTER(LincompRaggedDesc), _vp, _vp, _vp, _vp, _vp, _vp]
_lib.lincomp_run_ex.argtypes = [ctypes.POINTER(LincompDesc), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.lincomp_ragged_run_ex.argtypes = [ctypes.POINTER(LincompRaggedDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
for _f in ("gemm_plan_create", "gemm_plan_workspace_size", "gemm_plan_describe", "gemm_run", "gemm_run_ex",
           "gemm_run_noalloc", "gemm_plan_destroy", "lincomp_workspace_size", "lincomp_run", "lincomp_ragged_run",
           "lincomp_run_ex", "lincomp_ragged_run_ex"):
    getattr(_lib, _f).restype = ctypes.c_int


class LLError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {ll_status_string(status)}: {ll_last_error()}")


def ll_status_string(status: int) -> str:
    return _lib.ll_status_string(int(status)).decode()


def ll_last_error() -> str:
    return _lib.ll_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != LL_OK:
        raise LLError(status, what)


# ---------------------------------------------------------------------------
# C-ABI mirrors (pointers are ints; stream is a hipStream_t value or 0)
# ---------------------------------------------------------------------------

def gemm_plan_create(desc: GemmDesc) -> int:
    h = _vp()
    _check(_lib.gemm_plan_create(ctypes.byref(h), ctypes.byref(desc)), "gemm_plan_create")
    return h.value


def gemm_plan_workspace_size(plan: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.gemm_plan_workspace_size(plan, ctypes.byref(n)), "gemm_plan_workspace_size")
    return n.value


def gemm_plan_describe(plan: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(_lib.gemm_plan_describe(plan, buf, 512), "gemm_plan_describe")
    return buf.value.decode()


def gemm_run(plan: int, A: int, B: int, C: int, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(_lib.gemm_run(plan, A, B, C, workspace, ws_bytes, stream), "gemm_run")


def gemm_run_ex(plan: int, A: int, B: int, C: int, bias: int, workspace: int, ws_bytes: int,
                stream: int = 0) -> None:
    _check(_lib.gemm_run_ex(plan, A, B, C, bias, workspace, ws_bytes, stream), "gemm_run_ex")


LL_NOALLOC_SCRATCH_BYTES = 64 << 20


def gemm_run_noalloc(plan: int, A: int, B: int, C: int, bias: int | None = None, stream: int = 0) -> None:
    _check(_lib.gemm_run_noalloc(plan, A, B, C, bias, stream), "gemm_run_noalloc")


def gemm_plan_destroy(plan: int) -> None:
    _check(_lib.gemm_plan_destroy(plan), "gemm_plan_destroy")


def lincomp_workspace_size(desc: LincompDesc) -> int:
    n = ctypes.c_size_t()
    _check(_lib.lincomp_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "lincomp_workspace_size")
    return n.value


def lincomp_ragged_run(desc: LincompRaggedDesc, offsets: int, user: int, item: int, W: int, Y: int,
                       stream: int = 0) -> None:
    _check(_lib.lincomp_ragged_run(ctypes.byref(desc), offsets, user, item, W, Y, stream), "lincomp_ragged_run")


def lincomp_run(desc: LincompDesc, user: int, item: int, W: int, Y: int, workspace: int, ws_bytes: int,
                stream: int) -> None:
    _check(_lib.lincomp_run(ctypes.byref(desc), user, item, W, Y, workspace, ws_bytes, stream), "lincomp_run")


def lincomp_run_ex(desc: LincompDesc, user: int, item: int, W: int, bias: int | None, Y: int, workspace: int,
                   ws_bytes: int, stream: int) -> None:
    _check(_lib.lincomp_run_ex(ctypes.byref(desc), user, item, W, bias, Y, workspace, ws_bytes, stream),
           "lincomp_run_ex")


def lincomp_ragged_run_ex(desc: LincompRaggedDesc, offsets: int, user: int, item: int, W: int, bias: int | None,
                          Y: int, stream: int = 0) -> None:
    _check(_lib.lincomp_ragged_run_ex(ctypes.byref(desc), offsets, user, item, W, bias, Y, stream),
           "lincomp_ragged_run_ex")


# ---------------------------------------------------------------------------
# torch conveniences: build descriptors from tensor shapes/strides, keep plans
# and workspaces, launch on torch's current stream.
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return LL_BF16
    if dt == torch.float32:
        return LL_F32
    if dt == torch.float16:
        return LL_F16
    raise TypeError(f"unsupported dtype {dt}")


class GemmPlan:
    """Owns one gemm_plan and its workspaces on the plan's device: one per
    stream the plan runs on, so that runs on different streams never share
    packed copies or split-K partials (the C ABI asks concurrent runs for
    distinct workspaces)."""

    def __init__(self, desc: GemmDesc, device):
        self.desc = desc
        self.handle = gemm_plan_create(desc)
        self.ws_bytes = gemm_plan_workspace_size(self.handle)
        self.device = device
        torch = _torch()
        self._ws = {}
        # workspace of the stream current at creation (also what callers of
        # the raw C-ABI mirrors may pass)
        self.workspace = self.workspace_for(torch.cuda.current_stream(device).cuda_stream)

    def workspace_for(self, stream: int):
        ws = self._ws.get(stream)
        if ws is None:
            ws = _torch().empty(max(self.ws_bytes, 1), dtype=_torch().uint8, device=self.device)
            self._ws[stream] = ws
        return ws

    def describe(self) -> str:
        return gemm_plan_describe(self.handle)

    def run(self, A, B, C, stream: int | None = None, bias=None) -> None:
        if stream is None:
            stream = _torch().cuda.current_stream(A.device).cuda_stream
        ws = self.workspace_for(stream)
        if bias is not None or (self.desc.epilogue & LL_EPI_BIAS):
            gemm_run_ex(self.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                        bias.data_ptr() if bias is not None else None, ws.data_ptr(), self.ws_bytes, stream)
        else:
            gemm_run(self.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), ws.data_ptr(), self.ws_bytes, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:  # _lib is None once the interpreter tears the module down
            _lib.gemm_plan_destroy(h)
            self.handle = None


_plans: dict = {}


def gemm_desc_for(A, B, C, flags: int = 0, epilogue: int = 0) -> GemmDesc:
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    sa, sb, sc = A.stride(), B.stride(), C.stride()
    return GemmDesc(M, N, K, sa[0], sa[1], sb[0], sb[1], sc[0], sc[1],
                    _dtype_code(A.dtype), _dtype_code(B.dtype), _dtype_code(C.dtype), flags, epilogue)


def plan_for(A, B, C, flags: int = 0, epilogue: int = 0) -> GemmPlan:
    desc = gemm_desc_for(A, B, C, flags, epilogue)
    key = (A.device.index, tuple(getattr(desc, f) for f, _ in GemmDesc._fields_))
    plan = _plans.get(key)
    if plan is None:
        plan = GemmPlan(desc, A.device)
        _plans[key] = plan
    return plan


def gemm(A, B, out=None, out_dtype=None, flags: int = 0, bias=None, act=None):
    """C = act(A @ B + bias) for 2-D bf16 (or both fp16) CUDA (HIP) tensors with
    any row/column-major strides; C is bf16 (default), fp16 or fp32.  bias:
    optional fp32 [N]; act: None, "relu", "gelu" (exact) or "silu", applied
    to the fp32 sums in the GEMM's epilogue."""
    torch = _torch()
    if out is None:
        out = torch.empty((A.shape[0], B.shape[1]), dtype=out_dtype or torch.bfloat16, device=A.device)
    epilogue = ACTIVATIONS[act]
    if bias is not None:
        if bias.dtype != torch.float32 or tuple(bias.shape) != (B.shape[1],) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 tensor of N values")
        epilogue |= LL_EPI_BIAS
    plan_for(A, B, out, flags, epilogue).run(A, B, out, bias=bias)
    return out


def _lc_epilogue(bias, act, Mo) -> int:
    torch = _torch()
    epilogue = ACTIVATIONS[act]
    if bias is not None:
        if bias.dtype != torch.float32 or tuple(bias.shape) != (Mo,) or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous fp32 tensor of Mo values")
        epilogue |= LL_EPI_BIAS
    return epilogue


def lincomp_desc_for(user, item, W, Y, flags: int = 0, epilogue: int = 0) -> LincompDesc:
    """user is [R][Nu][D] (one block per request) or [R][C][Nu][D] (rows per
    candidate, e.g. the first Nu rows of a materialised input)."""
    R2, C, Ni, D2 = item.shape
    if user.dim() == 4:
        if user.shape[1] != C:
            raise ValueError("lincomp shape mismatch")
        R, _, Nu, D = user.shape
        su_r, su_c, su_n = user.stride(0), user.stride(1), user.stride(2)
    else:
        R, Nu, D = user.shape
        su_r, su_c, su_n = user.stride(0), 0, user.stride(1)
    Nin, Mo = W.shape
    if R2 != R or D2 != D or Nin != Nu + Ni or tuple(Y.shape) != (R, C, Mo, D):
        raise ValueError("lincomp shape mismatch")
    for t in (user, item, W, Y):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    si, sw, sy = item.stride(), W.stride(), Y.stride()
    return LincompDesc(R, C, Nu, Ni, D, Mo, su_r, su_c, su_n, si[0], si[1], si[2], sw[0],
                       sy[0], sy[1], sy[2], _dtype_code(Y.dtype), flags, epilogue)


_lc_ws: dict = {}


def lincomp(user, item, W, out=None, out_dtype=None, flags: int = 0, bias=None, act=None):
    """Y[r, c] = act(W^T . [user[r]; item[r, c]] + bias) for bf16 tensors user
    [R][Nu][D] (or [R][C][Nu][D], rows per candidate), item [R][C][Ni][D], W
    [Nu+Ni][Mo]; returns Y [R][C][Mo][D].  bias: optional fp32 [Mo], one per
    compressed row; act: None, "relu", "gelu" (exact) or "silu", applied to
    the fp32 sums before they are rounded."""
    torch = _torch()
    R, D = user.shape[0], user.shape[-1]
    C = item.shape[1]
    Mo = W.shape[1]
    if out is None:
        out = torch.empty((R, C, Mo, D), dtype=out_dtype or torch.bfloat16, device=user.device)
    desc = lincomp_desc_for(user, item, W, out, flags, _lc_epilogue(bias, act, Mo))
    need = lincomp_workspace_size(desc)
    key = user.device.index
    ws = _lc_ws.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=user.device)
        _lc_ws[key] = ws
    stream = torch.cuda.current_stream(user.device).cuda_stream
    lincomp_run_ex(desc, user.data_ptr(), item.data_ptr(), W.data_ptr(),
                   bias.data_ptr() if bias is not None else None, out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    return out



def lincomp_stacked(X, W, Nu: int, out=None, out_dtype=None, bias=None, act=None):
    """The layer's original form: X [R][C][Nu+Ni][D] holds every candidate's
    stacked input [user rows; item rows] in full.  Y[r, c] = act(W^T . X[r, c]
    + bias); each candidate computes its user rows' contribution itself."""
    return lincomp(X[:, :, :Nu], X[:, :, Nu:], W, out=out, out_dtype=out_dtype, bias=bias, act=act)


def lincomp_ragged(user, item, W, offsets, out=None, out_dtype=None, flags: int = 0, bias=None, act=None):
    """Ragged requests: user [R][Nu][D], item [Ctot][Ni][D], W [Nu+Ni][Mo] (bf16),
    offsets int64 [R+1] on the device (request r owns candidates
    offsets[r] .. offsets[r+1]-1); returns Y [Ctot][Mo][D]."""
    torch = _torch()
    R, Nu, D = user.shape
    Ctot, Ni, D2 = item.shape
    Nin, Mo = W.shape
    if D2 != D or Nin != Nu + Ni or tuple(offsets.shape) != (R + 1,) or offsets.dtype != torch.int64:
        raise ValueError("lincomp_ragged shape mismatch")
    if out is None:
        out = torch.empty((Ctot, Mo, D), dtype=out_dtype or torch.bfloat16, device=user.device)
    if tuple(out.shape) != (Ctot, Mo, D):
        raise ValueError("lincomp_ragged output shape mismatch")
    for t in (user, item, W, out):
        if t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    if not offsets.is_contiguous():
        raise ValueError("offsets must be contiguous")
    su, si, sw, sy = user.stride(), item.stride(), W.stride(), out.stride()
    desc = LincompRaggedDesc(R, Ctot, Nu, Ni, D, Mo, su[0], su[1], si[0], si[1], sw[0], sy[0], sy[1],
                             _dtype_code(out.dtype), flags, _lc_epilogue(bias, act, Mo))
    stream = torch.cuda.current_stream(user.device).cuda_stream
    lincomp_ragged_run_ex(desc, offsets.data_ptr(), user.data_ptr(), item.data_ptr(), W.data_ptr(),
                          bias.data_ptr() if bias is not None else None, out.data_ptr(), stream)
    return out
