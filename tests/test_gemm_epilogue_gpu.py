"""Fused GEMM epilogue (per-column fp32 bias, then ReLU / GELU / SiLU on the
fp32 sums) on the GPU against the fp64 oracle's epilogue."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, per_tile_indices, plan_tile, sample_indices, strip_starts, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _bias(N, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(N) * scale).astype(np.float32)


def _run(case, bias, act, flags=0):
    import torch
    import recsys_linear_layers_amd as ll
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    C = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    b = torch.from_numpy(bias).cuda() if bias is not None else None
    ll.gemm(A, B, out=C, flags=flags, bias=b, act=act)
    torch.cuda.synchronize()
    return to_f64(C)


def _check(case, bias, act):
    got = _run(case, bias, act)
    ref, S = oracle.gemm_case(case)
    ref, S = oracle.epilogue(ref, S, bias, act)
    acceptance.assert_close(got, ref, S, case.out_dtype, f"{case.name} act={act}", act=act)
    return got


@pytest.mark.parametrize("act", [None, "relu", "gelu", "silu"])
@pytest.mark.parametrize("M,N,K", [(257, 263, 300), (130, 1030, 520), (300, 8, 1000), (520, 264, 136)])
def test_bias_and_activation(act, M, N, K):
    c = synth.gemm_case(M, N, K, seed=M + 3 * N + 7 * K, out_dtype="f32")
    bias = _bias(N, M + N)
    _check(c, bias, act)
    c.out_dtype = "bf16"
    _check(c, bias, act)


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_activation_without_bias(act):
    c = synth.gemm_case(256, 512, 384, seed=31, out_dtype="f32")
    _check(c, None, act)


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_activation_accuracy_on_exact_sums(act):
    # Integer inputs make every fp32 sum exact, so only the activation's fp32
    # evaluation differs from the fp64 value: it must stay within 5e-7 |z| + 1e-6
    # (a tanh-form GELU, for one, is off by ~1e-4 near |z| = 1..3).
    c = synth.gemm_case(256, 256, 64, dist=("int", -1, 1), seed=32, out_dtype="f32")
    bias = np.round(_bias(256, 33, 2.0) * 8) / 8  # exact in fp32, sums stay exact
    bias = bias.astype(np.float32)
    got = _run(c, bias, act)
    z, _ = oracle.gemm_case(c)
    z = z + bias.astype(np.float64)
    ref, _ = oracle.epilogue(z, None, None, act)
    err = np.abs(got - ref)
    assert np.all(err <= 5e-7 * np.abs(z) + 1e-6), float(np.max(err / (5e-7 * np.abs(z) + 1e-6)))
    if act == "relu":
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_every_layout(la, lb):
    M, N, K = 200, 136, 72
    c = synth.gemm_case(M, N, K, seed=34, b_col_major=(lb == "col"), out_dtype="f32")
    if la == "col":
        c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=34, tensor=5)
        c.sam, c.sak = 1, M
    _check(c, _bias(N, 35), "silu")


def test_split_k_reduce_applies_epilogue():
    c = synth.gemm_case(128, 1024, 8192, seed=36, out_dtype="f32")
    _check(c, _bias(1024, 37), "gelu")
    c.out_dtype = "bf16"
    _check(c, _bias(1024, 37), "relu")


@pytest.mark.parametrize("N", [1024, 1030])
def test_split_k_reduce_store_paths_agree(N):
    """With N a multiple of 4 the split-K reduce takes four columns per thread
    and one 16-byte store into a row-major fp32 C, element stores into a
    column-major one; with N = 1030 every element goes through the per-element
    reduce.  Both C layouts give the same bits, matching the oracle."""
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.gemm_case(128, N, 8192, seed=38, out_dtype="f32", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    bias = torch.from_numpy(_bias(N, 39)).cuda()
    C1 = torch.full((128, N), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((N, 128), float("nan"), dtype=torch.float32, device="cuda").t()
    for C in (C1, C2):
        ll.gemm(A, B, out=C, bias=bias, act="silu")
    torch.cuda.synchronize()
    d = ll.plan_for(A, B, C1, 0, ll.LL_EPI_BIAS | ll.ACTIVATIONS["silu"]).describe()
    assert "splitk=1 " not in d, d
    g1, g2 = to_f64(C1), to_f64(C2)
    assert np.array_equal(g1, g2), d
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), "silu")
    acceptance.assert_close(g1, ref, S, "f32", f"split-K reduce N={N} {d}", act="silu")


def test_k_zero_gives_activation_of_bias():
    import torch
    import recsys_linear_layers_amd as ll
    bias = _bias(7, 38, 3.0)
    for act in (None, "relu", "gelu", "silu"):
        A = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
        B = torch.zeros((0, 7), dtype=torch.bfloat16, device="cuda")
        C = torch.full((5, 7), float("nan"), dtype=torch.float32, device="cuda")
        ll.gemm(A, B, out=C, bias=torch.from_numpy(bias).cuda(), act=act)
        torch.cuda.synchronize()
        ref, S = oracle.epilogue(np.zeros((5, 7)), np.zeros((5, 7)), bias, act)
        acceptance.assert_close(to_f64(C), ref, S, "f32", f"K=0 {act}", act=act)


def test_f16_operands_gelu_f16_out():
    c = synth.gemm_case(257, 263, 300, seed=39, in_dtype="f16", out_dtype="f16")
    _check(c, _bias(263, 40), "gelu")


def test_errors():
    import torch
    import recsys_linear_layers_amd as ll
    A = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    plan = ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.LL_EPI_GELU)
    with pytest.raises(ll.LLError):  # the plan adds a bias: plain gemm_run is refused
        ll.gemm_run(plan.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), plan.workspace.data_ptr(),
                    plan.ws_bytes, 0)
    with pytest.raises(ll.LLError):  # null bias
        ll.gemm_run_ex(plan.handle, A.data_ptr(), B.data_ptr(), C.data_ptr(), None, plan.workspace.data_ptr(),
                       plan.ws_bytes, 0)
    with pytest.raises(ll.LLError):  # cooperative kernels have no fused epilogue
        ll.plan_for(A, B, C, ll.LL_FLAG_COOPERATIVE, ll.LL_EPI_RELU)
    with pytest.raises(ll.LLError):  # unknown epilogue bits
        ll.plan_for(A, B, C, 0, 0x40)


def test_ffn_up_bias_gelu_sampled():
    """Full size: 4096 seeded entries (with the last tile row and column), one
    entry in every output tile of the plan's grid, a seeded 64-row strip and
    the first and last rows."""
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.gemm_workload("ffn_up")
    bias = _bias(c.N, 41, 0.5)
    got = _run(c, bias, "gelu")
    A, B = gemm_operands(c)
    C = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    tile = plan_tile(ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.LL_EPI_GELU).describe())
    del A, B, C
    rows, cols = sample_indices(c.M, c.N, 4096, seed=42, tile=tile)
    tr, tc = per_tile_indices(c.M, c.N, tile, 43)
    rows, cols = np.concatenate([rows, tr]), np.concatenate([cols, tc])
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    ref, S = oracle.epilogue(ref, S, bias, "gelu", cols=cols)
    acceptance.assert_close(got[rows, cols], ref, S, "bf16", f"ffn_up gelu samples (tile {tile})", act="gelu")
    for r0, nr in strip_starts(c.M, 64, 44):
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        ref, S = oracle.epilogue(ref, S, bias, "gelu")
        acceptance.assert_close(got[r0:r0 + nr], ref, S, "bf16", f"ffn_up gelu rows {r0}..{r0 + nr - 1}",
                                act="gelu")
