"""The C ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host (no GPU needed for these checks)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linlayers.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ll_status|const char\s*\*)\s*(\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("gemm_plan_create", "gemm_plan_workspace_size", "gemm_plan_describe", "gemm_run", "gemm_run_ex",
              "gemm_plan_destroy", "lincomp_workspace_size", "lincomp_run", "lincomp_ragged_run",
              "ll_status_string", "ll_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import recsys_linear_layers_amd as ll
    lib = ctypes.CDLL(ll.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings():
    import recsys_linear_layers_amd as ll
    assert ll.ll_status_string(ll.LL_OK) == "LL_OK"
    assert ll.ll_status_string(ll.LL_ERR_WORKSPACE) == "LL_ERR_WORKSPACE"
    assert ll.ll_status_string(ll.LL_ERR_NO_DEVICE) == "LL_ERR_NO_DEVICE"
    assert ll.ll_status_string(99) == "LL_ERR_UNKNOWN"


def _desc(**kw):
    import recsys_linear_layers_amd as ll
    base = dict(M=64, N=64, K=64, stride_am=64, stride_ak=1, stride_bk=64, stride_bn=1, stride_cm=64,
                stride_cn=1, a_type=ll.LL_BF16, b_type=ll.LL_BF16, c_type=ll.LL_F32, flags=0)
    base.update(kw)
    return ll.GemmDesc(**base)


def _create_status(desc):
    import recsys_linear_layers_amd as ll
    h = ctypes.c_void_p()
    st = ll._lib.gemm_plan_create(ctypes.byref(h), ctypes.byref(desc))
    if h.value:
        ll._lib.gemm_plan_destroy(h)
    return st


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.parametrize("kw,expect", [
    (dict(M=-1), "LL_ERR_INVALID_ARG"),
    (dict(K=-5), "LL_ERR_INVALID_ARG"),
    (dict(stride_am=0), "LL_ERR_INVALID_ARG"),
    (dict(stride_cn=-1), "LL_ERR_INVALID_ARG"),
    (dict(flags=0x100), "LL_ERR_INVALID_ARG"),
    (dict(flags=0x4 | 0x8), "LL_ERR_INVALID_ARG"),
    (dict(a_type=1), "LL_ERR_UNSUPPORTED"),
    (dict(c_type=7), "LL_ERR_UNSUPPORTED"),
    (dict(stride_am=64, stride_ak=2), "LL_ERR_UNSUPPORTED"),
    (dict(stride_bk=3, stride_bn=5), "LL_ERR_UNSUPPORTED"),
    (dict(M=1 << 31), "LL_ERR_UNSUPPORTED"),
    (dict(N=1 << 31), "LL_ERR_UNSUPPORTED"),
    (dict(K=1 << 23, stride_am=1 << 23), "LL_ERR_UNSUPPORTED"),   # K too large for 32-bit tile offsets
    (dict(a_type=2), "LL_ERR_UNSUPPORTED"),                        # fp16 A with bf16 B
    (dict(a_type=2, b_type=2, c_type=3), "LL_ERR_UNSUPPORTED"),
    (dict(epilogue=0x2), "LL_ERR_INVALID_ARG"),
    (dict(epilogue=0x40), "LL_ERR_INVALID_ARG"),
    (dict(epilogue=0x100), "LL_ERR_INVALID_ARG"),
])
def test_plan_argument_checks(kw, expect):
    import recsys_linear_layers_amd as ll
    assert ll.ll_status_string(_create_status(_desc(**kw))) == expect


def test_plan_null_arguments():
    import recsys_linear_layers_amd as ll
    assert ll._lib.gemm_plan_create(None, None) == ll.LL_ERR_INVALID_ARG
    assert "null" in ll.ll_last_error()
    h = ctypes.c_void_p()
    assert ll._lib.gemm_plan_create(ctypes.byref(h), None) == ll.LL_ERR_INVALID_ARG
    assert ll._lib.gemm_run(None, None, None, None, None, 0, None) == ll.LL_ERR_INVALID_ARG
    assert ll._lib.gemm_run_noalloc(None, None, None, None, None, None) == ll.LL_ERR_INVALID_ARG
    assert ll._lib.gemm_plan_workspace_size(None, None) == ll.LL_ERR_INVALID_ARG


def test_valid_plan_needs_a_device():
    import recsys_linear_layers_amd as ll
    st = _create_status(_desc())
    if _has_gpu():
        assert st == ll.LL_OK
    else:
        assert st == ll.LL_ERR_NO_DEVICE


def _lc(**kw):
    import recsys_linear_layers_amd as ll
    R, C, Nu, Ni, D, Mo = 2, 3, 256, 256, 256, 64
    base = dict(R=R, C=C, Nu=Nu, Ni=Ni, D=D, Mo=Mo, su_r=Nu * D, su_c=0, su_n=D, si_r=C * Ni * D, si_c=Ni * D,
                si_n=D, sw_n=Mo, sy_r=C * Mo * D, sy_c=Mo * D, sy_m=D, y_type=ll.LL_BF16, flags=0)
    base.update(kw)
    return ll.LincompDesc(**base)


def test_lincomp_workspace_and_checks():
    import recsys_linear_layers_amd as ll
    # the fused kernel keeps the per-request user contribution in registers
    assert ll.lincomp_workspace_size(_lc()) == 0
    assert ll.lincomp_workspace_size(_lc(flags=ll.LL_LINCOMP_NO_DEDUP)) == 0
    assert ll.lincomp_workspace_size(_lc(Nu=0)) == 0
    n = ctypes.c_size_t()
    for kw in (dict(R=-1), dict(D=12), dict(su_n=12), dict(flags=8), dict(y_type=5), dict(si_c=4),
               dict(sw_n=8), dict(sy_m=260), dict(su_c=4), dict(su_c=-8)):
        st = ll._lib.lincomp_workspace_size(ctypes.byref(_lc(**kw)), ctypes.byref(n))
        assert st != ll.LL_OK, kw
    st = ll._lib.lincomp_run(None, None, None, None, None, None, 0, None)
    assert st == ll.LL_ERR_INVALID_ARG


def _rg(**kw):
    import recsys_linear_layers_amd as ll
    R, Ctot, Nu, Ni, D, Mo = 3, 10, 64, 64, 64, 16
    base = dict(R=R, Ctot=Ctot, Nu=Nu, Ni=Ni, D=D, Mo=Mo, su_r=Nu * D, su_n=D, si_c=Ni * D, si_n=D, sw_n=Mo,
                sy_c=Mo * D, sy_m=D, y_type=ll.LL_BF16, flags=0)
    base.update(kw)
    return ll.LincompRaggedDesc(**base)


def test_ragged_argument_checks():
    import recsys_linear_layers_amd as ll
    run = ll._lib.lincomp_ragged_run
    assert run(None, None, None, None, None, None, None) == ll.LL_ERR_INVALID_ARG
    # null offsets with candidates to compute
    assert run(ctypes.byref(_rg()), None, 16, 16, 16, 16, None) == ll.LL_ERR_INVALID_ARG
    assert "offsets" in ll.ll_last_error()
    for kw in (dict(R=-1), dict(D=12), dict(si_c=4), dict(su_r=-8), dict(flags=8), dict(y_type=7),
               dict(sy_m=32)):
        st = run(ctypes.byref(_rg(**kw)), 16, 16, 16, 16, 16, None)
        assert st != ll.LL_OK, kw
    # nothing to compute: no device needed
    assert run(ctypes.byref(_rg(R=0, Ctot=0)), None, None, None, None, None, None) == ll.LL_OK


def test_gemm_run_ex_null_plan():
    import recsys_linear_layers_amd as ll
    assert ll._lib.gemm_run_ex(None, None, None, None, None, None, 0, None) == ll.LL_ERR_INVALID_ARG


PROBE_HEADER = os.path.join(ROOT, "include", "llprobes.h")
PROBE_LIB = os.path.join(ROOT, "recsys_linear_layers_amd", "libllprobes.so")


def _probe_lib():
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ll_probe_mfma_only.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ll_probe_mfma16_only.argtypes = lib.ll_probe_mfma_only.argtypes
    lib.ll_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.ll_probe_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_void_p]
    return lib


def test_probe_library_exports_every_declared_symbol():
    names = re.findall(r"^int\s+(\w+)\s*\(", open(PROBE_HEADER).read(), re.M)
    assert sorted(names) == ["ll_probe_mfma16_only", "ll_probe_mfma_only", "ll_probe_read", "ll_probe_stream"]
    lib = ctypes.CDLL(PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_probes_reject_bad_arguments_on_the_host():
    """Every rejected call returns -1 before any HIP call is made."""
    lib = _probe_lib()
    for f in (lib.ll_probe_mfma_only, lib.ll_probe_mfma16_only):
        assert f(0, 10, None, 256, None) == -1    # grid < 1
        assert f(1, -1, None, 256, None) == -1    # iters < 0
        assert f(1, 10, None, None, None) == -1   # no output
        assert f(1, 10, 4100, 256, None) == -1    # misaligned operands
    assert lib.ll_probe_stream(2, 0, 4096, 1 << 20, 16, 1, None) == -1  # streams not 1 or 4
    assert lib.ll_probe_stream(1, 4, 4096, 1 << 20, 16, 1, None) == -1  # unknown hint bits
    assert lib.ll_probe_stream(1, 0, 4096, 1 << 20, -1, 1, None) == -1  # n16 < 0
    assert lib.ll_probe_stream(1, 0, 4096, 1 << 20, 16, 0, None) == -1  # grid < 1
    assert lib.ll_probe_stream(1, 0, 4100, 1 << 20, 16, 1, None) == -1  # misaligned x
    assert lib.ll_probe_stream(4, 3, 4096, 4096 + 16 * 16, 16, 1, None) == -1  # y inside x
    assert lib.ll_probe_stream(1, 3, None, None, 0, 1, None) == 0     # nothing to do
    assert lib.ll_probe_read(2, 4096, 1 << 20, 16, 1, None) == -1      # unknown hint bits
    assert lib.ll_probe_read(0, 4096, 1 << 20, -1, 1, None) == -1      # n16 < 0
    assert lib.ll_probe_read(0, 4096, 1 << 20, 16, 0, None) == -1      # grid < 1
    assert lib.ll_probe_read(0, 4096, None, 16, 1, None) == -1         # no y
    assert lib.ll_probe_read(0, 4104, 1 << 20, 16, 1, None) == -1      # misaligned x
    assert lib.ll_probe_read(1, 4096, 4096 + 16 * 8, 16, 1, None) == -1  # y inside x
