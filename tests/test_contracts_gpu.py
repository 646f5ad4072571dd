"""Contracts of the C ABI on the GPU: overlap rejection, workspace checks, and
concurrent runs of one plan on two streams (plans are immutable; each run
brings its own workspace)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, lincomp_operands, strip_starts, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def test_c_overlapping_an_operand_is_rejected():
    import torch
    import recsys_linear_layers_amd as ll
    buf = torch.zeros(2 * 64 * 64, dtype=torch.bfloat16, device="cuda")
    A = buf[: 64 * 64].view(64, 64)
    B = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    C = buf[32 * 64: 96 * 64].view(64, 64)  # shares half its rows with A
    with pytest.raises(ll.LLError) as e:
        ll.gemm(A, B, out=C)
    assert e.value.status == ll.LL_ERR_INVALID_ARG


def test_y_overlapping_an_input_is_rejected():
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.lincomp_case(2, 3, 64, 64, 64, 16, seed=80, name="ov")
    user, item, W = lincomp_operands(c)
    Y = item.reshape(-1)[: 2 * 3 * 16 * 64].view(2, 3, 16, 64)  # Y inside item
    with pytest.raises(ll.LLError) as e:
        ll.lincomp(user, item, W, out=Y)
    assert e.value.status == ll.LL_ERR_INVALID_ARG


def test_split_k_workspace_too_small_is_rejected():
    import torch
    import recsys_linear_layers_amd as ll
    A = torch.zeros((128, 65536), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((65536, 1024), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((128, 1024), dtype=torch.float32, device="cuda")
    plan = ll.plan_for(A, B, C)
    assert plan.ws_bytes > 0 and "splitk=1 " not in plan.describe()
    with pytest.raises(ll.LLError) as e:
        ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), plan.workspace.data_ptr(),
                    plan.ws_bytes - 1, 0)
    assert e.value.status == ll.LL_ERR_WORKSPACE


def test_misaligned_workspace_is_rejected():
    import torch
    import recsys_linear_layers_amd as ll
    # column-major B with an odd leading dimension: packed (K-contiguous, beside a K-contiguous A) into the workspace
    A = torch.zeros((300, 520), dtype=torch.bfloat16, device="cuda")
    Bt = torch.zeros((260, 521), dtype=torch.bfloat16, device="cuda")[:, :520]
    B = Bt.t()
    C = torch.zeros((300, 260), dtype=torch.float32, device="cuda")
    plan = ll.plan_for(A, B, C)
    assert plan.ws_bytes > 0 and "packB=1" in plan.describe() and "B:K-major" in plan.describe()
    ws = torch.empty(plan.ws_bytes + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ll.LLError) as e:
        ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), ws.data_ptr() + 16, plan.ws_bytes, 0)
    assert e.value.status == ll.LL_ERR_WORKSPACE
    assert "aligned" in ll.ll_last_error()


def test_one_plan_two_streams_concurrently():
    import torch
    import recsys_linear_layers_amd as ll
    # split-K shape, so each run needs its own workspace
    c = synth.gemm_case(128, 1024, 8192, seed=81, out_dtype="f32")
    A, B = gemm_operands(c)
    C1 = torch.full((128, 1024), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((128, 1024), float("nan"), dtype=torch.float32, device="cuda")
    plan = ll.plan_for(A, B, C1)
    ws2 = torch.empty(max(plan.ws_bytes, 1), dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C1.data_ptr(), plan.workspace.data_ptr(),
                    plan.ws_bytes, s1.cuda_stream)
        ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C2.data_ptr(), ws2.data_ptr(), plan.ws_bytes,
                    s2.cuda_stream)
    torch.cuda.synchronize()
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C1), ref, S, "f32", "stream 1")
    assert torch.equal(C1, C2)  # same plan, same order of sums: bit-identical


@pytest.mark.parametrize("shape,b_col", [((128, 1024, 8192), False), ((300, 260, 520), True)])
def test_gemm_convenience_on_two_streams(shape, b_col):
    """ll.gemm on two streams at once with one cached plan (a split-K shape,
    and a column-major B with an odd leading dimension that is packed): each
    stream gets its own workspace, so neither run reads the other's partials or
    packed copy."""
    import torch
    import recsys_linear_layers_amd as ll
    M, N, K = shape
    cases = [synth.gemm_case(M, N, K, seed=82 + i, out_dtype="f32", b_col_major=b_col,
                             ldb=(K + 1 if b_col else None)) for i in range(2)]
    ops = [gemm_operands(c) for c in cases]
    outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for _ in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for (A, B), C, st in zip(ops, outs, streams):
            with torch.cuda.stream(st):
                ll.gemm(A, B, out=C)
    torch.cuda.synchronize()
    d = ll.plan_for(ops[0][0], ops[0][1], outs[0]).describe()
    assert ("splitk=1 " not in d) if not b_col else ("packB=1" in d), d
    for c, C in zip(cases, outs):
        ref, S = oracle.gemm_case(c)
        acceptance.assert_close(to_f64(C), ref, S, "f32", f"{c.name} seed on its own stream")


def test_plan_describe_reports_the_choice():
    import torch
    import recsys_linear_layers_amd as ll
    A = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    d = ll.plan_for(A, A, C).describe()
    assert "kernel=KIND_SQ4_HO" in d and "splitk=1" in d
    d = ll.plan_for(A, A, C, 0, ll.LL_EPI_GELU).describe()
    assert "fused=3" in d and "kernel=KIND_SQ4_HO" in d


def test_round_barrier_plans_on_two_streams(monkeypatch):
    """Two hand-ordered GEMMs with round barriers at once, on two streams: the
    second kernel's workgroups wait for CUs the first holds, so their round
    waits may run out.  The wait is bounded and changes no arithmetic: both
    results equal a run alone."""
    import torch
    import recsys_linear_layers_amd as ll
    M, N, K = 8192, 8192, 512
    c = synth.gemm_case(M, N, K, seed=99, out_dtype="bf16", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    outs = [torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "1")
    plan = ll.GemmPlan(ll.gemm_desc_for(A, B, outs[0]), A.device)
    monkeypatch.delenv("LL_GEMM_ROUND_SYNC")
    assert "kernel=KIND_SQ4_HO " in plan.describe() and "round_sync=1" in plan.describe(), plan.describe()
    plan.run(A, B, outs[2])
    torch.cuda.synchronize()
    wss = [torch.empty(plan.ws_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for C, ws, st in zip(outs[:2], wss, streams):
            ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), ws.data_ptr(), plan.ws_bytes,
                        st.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[2])
    for r0, nr in strip_starts(M, 64, 100):
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        acceptance.assert_close(to_f64(outs[2][r0:r0 + nr]), ref, S, "bf16", f"rows {r0}..")
