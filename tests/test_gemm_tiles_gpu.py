"""Tile-count quantisation and the 192x256 kind.

The plan replaces the 256x128 / 128x256 producer/consumer tiles by 192x256
tiles when those cover the problem in fewer passes over the CUs (A
K-contiguous only).  Parity against the fp64 oracle for shapes that select it
and for the kind forced on small ragged shapes, in every layout it supports;
the layouts it cannot load are refused."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, sample_indices, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu

KIND = "KIND_T192_PC"


def _ll():
    import recsys_linear_layers_amd as ll
    return ll


def _describe(M, N, K, a_col=False, b_col=False, in_t=None, c_t=None, flags=0, epilogue=0):
    ll = _ll()
    in_t = ll.LL_BF16 if in_t is None else in_t
    c_t = ll.LL_BF16 if c_t is None else c_t
    sam, sak = (1, M) if a_col else (K, 1)
    sbk, sbn = (1, K) if b_col else (N, 1)
    desc = ll.GemmDesc(M, N, K, sam, sak, sbk, sbn, N, 1, in_t, in_t, c_t, flags, epilogue)
    h = ll.gemm_plan_create(desc)
    try:
        return ll.gemm_plan_describe(h)
    finally:
        ll._lib.gemm_plan_destroy(h)


@pytest.fixture
def forced_kind(monkeypatch):
    """Force the 192x256 kind for plans made inside the test; cached plans are
    dropped before and after so that no forced plan outlives the test."""
    ll = _ll()
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    yield
    monkeypatch.delenv("LL_GEMM_KIND", raising=False)
    ll._plans.clear()


def _run(case, flags=0):
    import torch
    ll = _ll()
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    C = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    plan = ll.plan_for(A, B, C, flags)
    desc = plan.describe()
    plan.run(A, B, C)
    torch.cuda.synchronize()
    return C, desc


@pytest.mark.parametrize("M,N,K,want", [
    (2900, 2900, 136, True),      # 276 tiles of 256x128 (2 passes) vs 192 of 192x256 (1 pass)
    (3000, 3000, 3000, True),     # 288 tiles of 256x128 (2 passes) vs 192 of 192x256 (1 pass)
    (4000, 3000, 1000, True),     # 384 of 128x256 (2 passes) vs 252 of 192x256 (1 pass)
    (4096, 4096, 4096, False),    # 512 tiles of 256x128: 2 whole passes
    (16384, 28672, 8192, False),  # FFN up
    (16384, 8192, 28672, False),  # FFN down
    (8191, 5003, 4099, False),    # 1280 tiles: 5 whole passes
    (128, 8192, 65536, False),    # skinny: split-K
    (2048, 2048, 4096, False),    # few tiles: split-K, not the tile rule
])
def test_rule_selection(M, N, K, want):
    d = _describe(M, N, K)
    assert (KIND in d) == want, d


def test_rule_needs_k_contiguous_a_and_no_forced_mode():
    ll = _ll()
    # M = 2904 keeps a column-major A direct (M-contiguous); with M not a
    # multiple of 8 it would be packed into a K-contiguous copy, where the rule applies
    assert KIND in _describe(2904, 2900, 136)
    assert KIND not in _describe(2904, 2900, 136, a_col=True)
    assert KIND in _describe(2900, 2900, 136, a_col=True)
    assert KIND in _describe(2900, 2900, 136, b_col=True)
    assert KIND in _describe(2900, 2900, 136, in_t=ll.LL_F16, c_t=ll.LL_F16)
    assert KIND in _describe(2900, 2900, 136, epilogue=ll.LL_EPI_GELU)
    assert KIND in _describe(2900, 2900, 136, epilogue=ll.LL_EPI_BIAS | ll.LL_EPI_SILU)
    assert KIND not in _describe(2900, 2900, 136, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    assert KIND not in _describe(2900, 2900, 136, flags=ll.LL_FLAG_COOPERATIVE)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_selected_full_parity(out):
    # ragged in M (2900 = 15*192 + 20), N (11*256 + 84) and K (2*64 + 8)
    c = synth.gemm_case(2900, 2900, 136, seed=192, dist=("normal", 0.0, 1.0), out_dtype=out)
    C, desc = _run(c)
    assert KIND in desc, desc
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C), ref, S, out, f"2900x2900x136 {out}")


def test_gemm_3000_workload_sampled():
    """The benchmark's mid-size workload, at its full size, in the kind the rule picks."""
    c = synth.gemm_workload("gemm_3000")
    C, desc = _run(c)
    assert KIND in desc, desc
    got = to_f64(C)
    rows, cols = sample_indices(c.M, c.N, 4096, seed=4, tile=192)
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    acceptance.assert_close(got[rows, cols], ref, S, "bf16", "gemm_3000 samples")
    for r0 in (0, 2880, c.M - 8):   # first rows, the last row of tiles, the ragged end
        ref, S = oracle.gemm_case(c, rows=(r0, 8))
        acceptance.assert_close(got[r0:r0 + 8], ref, S, "bf16", f"gemm_3000 strip {r0}")


def test_selected_mid_shape_sampled():
    c = synth.gemm_case(4000, 3000, 1000, seed=193, dist=("normal", 0.0, 1.0), out_dtype="bf16")
    C, desc = _run(c)
    assert KIND in desc, desc
    got = to_f64(C)
    rows, cols = sample_indices(c.M, c.N, 4096, seed=3, tile=192)
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    acceptance.assert_close(got[rows, cols], ref, S, "bf16", "4000x3000x1000 samples")
    for r0 in (0, 3840, c.M - 8):   # first rows, the last row of tiles, the ragged end
        ref, S = oracle.gemm_case(c, rows=(r0, 8))
        acceptance.assert_close(got[r0:r0 + 8], ref, S, "bf16", f"4000x3000x1000 strip {r0}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 9, 13), (200, 136, 72), (257, 263, 300), (130, 1030, 520),
                                   (385, 513, 200)])
@pytest.mark.parametrize("lb", ["row", "col"])
@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
def test_forced_small_shapes(forced_kind, M, N, K, lb, in_dtype):
    seed = M * 7919 + N * 31 + K
    c = synth.gemm_case(M, N, K, seed=seed, b_col_major=(lb == "col"), out_dtype="f32", in_dtype=in_dtype)
    outs = ("f32", "bf16") if in_dtype == "bf16" else ("f32", "f16")
    for out in outs:
        c.out_dtype = out
        C, desc = _run(c)
        assert KIND in desc, desc
        ref, S = oracle.gemm_case(c)
        acceptance.assert_close(to_f64(C), ref, S, out, f"{M}x{N}x{K} B {lb} {in_dtype}->{out}")


def test_forced_integer_inputs_bit_exact(forced_kind):
    c = synth.gemm_case(520, 264, 1992, dist=("int", -4, 4), seed=17)
    C, desc = _run(c)
    assert KIND in desc, desc
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(to_f64(C), ref)


def test_forced_on_column_major_a_is_refused(forced_kind):
    ll = _ll()
    with pytest.raises(ll.LLError) as e:
        _describe(304, 300, 64, a_col=True)   # M % 8 == 0: A stays M-contiguous (no pack)
    assert e.value.status == ll.LL_ERR_UNSUPPORTED
    assert "K-contiguous" in ll.ll_last_error()


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_selected_fused_epilogue(act):
    """Bias + activation fused into the 192x256 kind, on a shape the rule selects."""
    import torch
    ll = _ll()
    c = synth.gemm_case(2900, 2900, 136, seed=194, dist=("normal", 0.0, 1.0), out_dtype="bf16")
    A, B = gemm_operands(c)
    bias = torch.linspace(-2.0, 2.0, c.N, dtype=torch.float32, device="cuda")
    C = torch.full((c.M, c.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ll.gemm(A, B, out=C, bias=bias, act=act)
    torch.cuda.synchronize()
    epi = ll.LL_EPI_BIAS | {"relu": ll.LL_EPI_RELU, "gelu": ll.LL_EPI_GELU, "silu": ll.LL_EPI_SILU}[act]
    assert KIND in ll.plan_for(A, B, C, 0, epi).describe()
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(to_f64(C), ref, S, "bf16", f"2900x2900x136 bias+{act}", act=act)


def test_forced_fused_epilogue_small(forced_kind):
    import torch
    ll = _ll()
    c = synth.gemm_case(257, 263, 300, seed=195, dist=("normal", 0.0, 1.0), out_dtype="f32")
    A, B = gemm_operands(c)
    bias = torch.linspace(-1.0, 1.0, c.N, dtype=torch.float32, device="cuda")
    C = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ll.gemm(A, B, out=C, bias=bias, act="gelu")
    torch.cuda.synchronize()
    assert KIND in ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.LL_EPI_GELU).describe()
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), "gelu")
    acceptance.assert_close(to_f64(C), ref, S, "f32", "257x263x300 bias+gelu forced", act="gelu")
