"""gemm_run_noalloc (the GEMM entry point that allocates nothing and keeps its
workspace in a device array inside the library) against gemm_run_ex with the
plan's own workspace, through the C ABI: results must be bit-identical (same
kernels, same order of sums), on two calls in a row, the second smaller, for
split-K partials, packed operand copies, the round counters and K-split
last rounds of the hand-ordered kind (with B N- or K-contiguous); plus the
size limit."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _pair(case, act=None, bias_seed=None):
    """(C from gemm_run_ex with the plan's workspace, C from gemm_run_noalloc, plan description)."""
    import torch
    import recsys_linear_layers_amd as ll
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[case.out_dtype]
    C_ref = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    C_na = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    epi = ll.ACTIVATIONS[act]
    bias = None
    if bias_seed is not None:
        bias = torch.from_numpy(np.random.default_rng(bias_seed).standard_normal(case.N).astype(np.float32)).cuda()
        epi |= ll.LL_EPI_BIAS
    plan = ll.GemmPlan(ll.gemm_desc_for(A, B, C_ref, 0, epi), A.device)
    assert 0 < plan.ws_bytes <= ll.LL_NOALLOC_SCRATCH_BYTES, plan.ws_bytes
    stream = torch.cuda.current_stream().cuda_stream
    bptr = bias.data_ptr() if bias is not None else None
    ll.gemm_run_ex(plan.handle, A.data_ptr(), B.data_ptr(), C_ref.data_ptr(), bptr, plan.workspace.data_ptr(),
                   plan.ws_bytes, stream)
    ll.gemm_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(), C_na.data_ptr(), bptr, stream)
    torch.cuda.synchronize()
    return C_ref, C_na, plan.describe(), (None if bias is None else bias.cpu().numpy())


def _check(case, act=None, bias_seed=None, want=""):
    C_ref, C_na, d, bias = _pair(case, act, bias_seed)
    assert want in d, d
    assert not torch_isnan_any(C_na)
    assert np.array_equal(to_f64(C_ref), to_f64(C_na)), f"{case.name}: noalloc differs from gemm_run_ex ({d})"
    ref, S = oracle.gemm_case(case)
    if act is not None or bias is not None:
        ref, S = oracle.epilogue(ref, S, bias, act)
    acceptance.assert_close(to_f64(C_na), ref, S, case.out_dtype, f"{case.name} noalloc ({d})", act=act)


def torch_isnan_any(t):
    import torch
    return bool(torch.isnan(t.float()).any())


def test_split_k_two_calls_second_smaller():
    # 16 split-K partials of 128x4096 fp32 (33.5 MB), then 16 of 128x1024 (8.4 MB)
    big = synth.gemm_case(128, 4096, 32768, seed=301, out_dtype="f32", name="noalloc_splitk_big")
    small = synth.gemm_case(128, 1024, 8192, seed=302, out_dtype="bf16", name="noalloc_splitk_small")
    _check(big, want="splitk=16 ")
    _check(small, act="relu", bias_seed=303, want="splitk=16 ")


def test_packed_operands_two_calls_second_smaller():
    # column-major A and column-major B with odd leading dimensions: both packed
    def case(M, N, K, seed, name):
        c = synth.gemm_case(M, N, K, seed=seed, b_col_major=True, ldb=K + 3, out_dtype="f32", name=name)
        c.A = synth.bf16_tensor((M + 5) * K, "uniform", -1.0, 1.0, seed=seed, tensor=5)
        c.sam, c.sak = 1, M + 5
        return c
    _check(case(1030, 777, 1301, 304, "noalloc_pack_big"), want="packA=1 packB=1")
    _check(case(300, 260, 519, 305, "noalloc_pack_small"), act="gelu", bias_seed=306, want="packA=1 packB=1")


def test_round_counters_two_calls_second_smaller(monkeypatch):
    # the hand-ordered kind with its round barrier: the counters sit in the
    # workspace and each call clears them first (2 rounds each: 306, then 289 tiles)
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "1")
    big = synth.gemm_case(4608, 4352, 128, seed=307, out_dtype="bf16", dist=("normal", 0.0, 1.0),
                          name="noalloc_rounds_big")
    small = synth.gemm_case(4352, 4160, 64, seed=308, out_dtype="bf16", dist=("normal", 0.0, 1.0),
                            name="noalloc_rounds_small")
    _check(big, want="round_sync=1")
    _check(small, act="silu", bias_seed=309, want="round_sync=1")


def test_tail_split_two_calls_second_smaller(monkeypatch):
    # the hand-ordered kind's K-split last round: partial tiles in the
    # workspace, then the reduce (289 tiles: 33 split 4 ways, then 2 ways)
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    big = synth.gemm_case(4352, 4160, 4096, seed=317, out_dtype="bf16", dist=("normal", 0.0, 1.0),
                          name="noalloc_tail_big")
    small = synth.gemm_case(4352, 4160, 2048, seed=318, out_dtype="f32", dist=("normal", 0.0, 1.0),
                            name="noalloc_tail_small")
    _check(big, want="tail=33x4")
    _check(small, act="gelu", bias_seed=319, want="tail=33x2")


def test_plan_beyond_the_scratch_size_is_refused():
    import torch
    import recsys_linear_layers_amd as ll
    # a K-contiguous A with K % 8 != 0 is packed into [8192][4160] bf16 (68.2 MB > 64 MiB)
    d = ll.GemmDesc(8192, 256, 4100, 4100, 1, 256, 1, 256, 1, ll.LL_BF16, ll.LL_BF16, ll.LL_F32, 0, 0)
    h = ll.gemm_plan_create(d)
    try:
        assert ll.gemm_plan_workspace_size(h) > ll.LL_NOALLOC_SCRATCH_BYTES
        dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
        st = ll._lib.gemm_run_noalloc(h, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), None, 0)
        assert st == ll.LL_ERR_WORKSPACE, ll.ll_status_string(st)
        assert "at most" in ll.ll_last_error()
    finally:
        ll.gemm_plan_destroy(h)


def test_b_k_contiguous_tail_split_two_calls_second_smaller(monkeypatch):
    # C = X W^T (B K-contiguous) in the hand-ordered kind, whose K-split last
    # round keeps its partials in the device array
    monkeypatch.delenv("LL_GEMM_TAIL_SPLIT", raising=False)
    big = synth.gemm_case(4352, 4160, 4096, seed=331, out_dtype="bf16", b_col_major=True, name="noalloc_nt_big")
    small = synth.gemm_case(4352, 4160, 2048, seed=332, out_dtype="f32", b_col_major=True, name="noalloc_nt_small")
    _check(big, want="B:K-major")
    _check(small, act="silu", bias_seed=333, want="tail=33x2")


def test_plan_without_workspace():
    # 4096^3 needs no workspace: the call runs straight through
    c = synth.gemm_case(1024, 1024, 512, seed=307, out_dtype="bf16", name="noalloc_plain")
    import torch
    import recsys_linear_layers_amd as ll
    A, B = gemm_operands(c)
    C1 = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    plan = ll.plan_for(A, B, C1)
    assert plan.ws_bytes == 0
    ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C1.data_ptr(), 0, 0, 0)
    ll.gemm_run_noalloc(plan.handle, A.data_ptr(), B.data_ptr(), C2.data_ptr(), None, 0)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
