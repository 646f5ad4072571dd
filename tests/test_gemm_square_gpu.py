"""The 256x256 kind with eight computing waves, one per SIMD also loading.

The plan puts it in place of the 256x128 producer/consumer tile when A is
K-contiguous, B is N-contiguous, there is no fused epilogue, and its tiles
cover the problem in no more passes times tile area; where K is a multiple of
64 the hand-ordered 256x256 kind (four 128x128 waves) takes its place again.
Parity against the fp64 oracle on ragged shapes that select it, the selection
on the benchmark shapes, and the kind forced on small ragged shapes in every
operand layout, both input types, split-K and K = 0."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, sample_indices, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu

KIND = "KIND_SQ8_LW4"


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
    """Force the 256x256 kind for plans made inside the test; cached plans are
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


SQ4 = "KIND_SQ4_HO"


@pytest.mark.parametrize("M,N,K,want", [
    (4096, 4096, 4096, SQ4),         # K a multiple of 64: the hand-ordered kind
    (16384, 28672, 8192, SQ4),       # FFN up
    (16384, 8192, 28672, SQ4),       # FFN down
    (8192, 8192, 28672, SQ4),
    (8192, 8192, 8192, SQ4),
    (4096, 4096, 4104, KIND),        # K not a multiple of 64: 256 tiles of 256x256 vs 512 of 256x128
    (4000, 4000, 136, KIND),         # ragged
    (16384, 28672, 8136, KIND),      # FFN up with K % 64 = 8
    (4096, 2048, 8192, "KIND_TALL_PC"),   # 128 tiles of 256x256 would split K; M > N
    (2048, 4096, 8192, "KIND_WIDE_PC"),   # same, M < N
    (3000, 3000, 3000, "KIND_T192_PC"),   # the 192x256 tile-count rule
    (128, 8192, 65536, "KIND_TALL_PC"),   # skinny: split-K
])
def test_rule_selection(M, N, K, want):
    d = _describe(M, N, K)
    assert f"kernel={want} " in d, d


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 28680), (4096, 4096, 16392), (8192, 16384, 24584)])
def test_long_k_rule_picks_128x256(M, N, K):
    # K > 8192 and not a multiple of 64 (else the hand-ordered kind takes it)
    ll = _ll()
    assert "kernel=KIND_TALL_PC " in _describe(M, N, K)
    # with a fused epilogue, another layout or a forced mode the rule stays out
    assert "kernel=KIND_TALL_PC " not in _describe(M, N, K, epilogue=ll.LL_EPI_GELU)
    assert "kernel=KIND_TALL_PC " not in _describe(M, N, K, b_col=True)


def test_long_k_selected_sampled():
    """A square long-K shape the rule sends to the 128x256 kind, at full size:
    sampled entries (the corners and the last tile row and column included)
    and row strips against the oracle."""
    c = synth.gemm_case(4096, 4096, 16392, seed=259, dist=("normal", 0.0, 1.0), out_dtype="bf16")
    C, desc = _run(c)
    assert "kernel=KIND_TALL_PC " in desc, desc
    got = to_f64(C)
    rows, cols = sample_indices(c.M, c.N, 2048, seed=6, tile=256)
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    acceptance.assert_close(got[rows, cols], ref, S, "bf16", "4096x4096x16392 samples")
    for r0 in (0, c.M - 8):
        ref, S = oracle.gemm_case(c, rows=(r0, 8))
        acceptance.assert_close(got[r0:r0 + 8], ref, S, "bf16", f"4096x4096x16392 strip {r0}")


def test_rule_conditions():
    ll = _ll()
    K = 4104  # not a multiple of 64, so the hand-ordered kind stays out
    assert KIND in _describe(4096, 4096, K, in_t=ll.LL_F16, c_t=ll.LL_F16)
    assert KIND in _describe(4096, 4096, K, c_t=ll.LL_F32)
    assert KIND not in _describe(4096, 4096, K, b_col=True)   # B K-contiguous
    assert KIND not in _describe(4096, 4096, K, a_col=True)   # A M-contiguous
    assert KIND not in _describe(4096, 4096, K, epilogue=ll.LL_EPI_GELU)
    assert KIND not in _describe(4096, 4096, K, epilogue=ll.LL_EPI_BIAS)
    assert KIND not in _describe(4096, 4096, K, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    assert KIND not in _describe(4096, 4096, K, flags=ll.LL_FLAG_COOPERATIVE)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_selected_full_parity(out):
    # ragged in M and N (4000 = 15*256 + 160) and K (2*64 + 8)
    c = synth.gemm_case(4000, 4000, 136, seed=256, dist=("normal", 0.0, 1.0), out_dtype=out)
    C, desc = _run(c)
    assert KIND in desc, desc
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C), ref, S, out, f"4000x4000x136 {out}")


def test_selected_integer_inputs_bit_exact():
    c = synth.gemm_case(4000, 4000, 520, dist=("int", -4, 4), seed=257, out_dtype="f32")
    C, desc = _run(c)
    assert KIND in desc, desc
    got = to_f64(C)
    rows, cols = sample_indices(c.M, c.N, 4096, seed=5, tile=256)
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(got[rows, cols], ref)
    for r0 in (0, 3840, c.M - 8):   # first rows, the last row of tiles, the ragged end
        ref, _ = oracle.gemm_case(c, rows=(r0, 8))
        assert np.array_equal(got[r0:r0 + 8], ref)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (7, 9, 13), (200, 136, 72), (257, 263, 300), (130, 1030, 520),
                                   (385, 513, 200), (600, 520, 1000)])
@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
@pytest.mark.parametrize("in_dtype", ["bf16", "f16"])
def test_forced_small_shapes(forced_kind, M, N, K, la, lb, in_dtype):
    seed = M * 7919 + N * 31 + K + (la == "col") * 3 + (lb == "col")
    c = synth.gemm_case(M, N, K, seed=seed, b_col_major=(lb == "col"), out_dtype="f32", in_dtype=in_dtype)
    if la == "col":  # re-describe A column-major: buffer is [K][M]
        c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=seed, tensor=5, fmt=in_dtype)
        c.sam, c.sak = 1, M
    outs = ("f32", "bf16") if in_dtype == "bf16" else ("f32", "f16")
    for out in outs:
        c.out_dtype = out
        C, desc = _run(c)
        assert KIND in desc, desc
        ref, S = oracle.gemm_case(c)
        acceptance.assert_close(to_f64(C), ref, S, out, f"{M}x{N}x{K} A {la} B {lb} {in_dtype}->{out}")


def test_forced_split_k_integer_exact(forced_kind):
    # 2 tiles of 256x256: the plan splits K; integer sums make every order exact
    c = synth.gemm_case(256, 400, 8200, dist=("int", -4, 4), seed=258, out_dtype="f32")
    C, desc = _run(c)
    assert KIND in desc and "splitk=1 " not in desc, desc
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(to_f64(C), ref)


def test_forced_k_zero(forced_kind):
    import torch
    ll = _ll()
    A = torch.zeros((300, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((0, 270), dtype=torch.bfloat16, device="cuda")
    C = torch.full((300, 270), float("nan"), dtype=torch.float32, device="cuda")
    ll.gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0
