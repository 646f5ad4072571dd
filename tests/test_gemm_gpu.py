"""GEMM parity on the GPU: the HIP path (through the C ABI) against the fp64
oracle, element by element within the acceptance bound, and bit-exact where
integer-valued inputs make every fp32 partial sum exact."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, per_tile_indices, plan_tile, sample_indices, strip_starts, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _ll():
    import recsys_linear_layers_amd as ll
    return ll


def _run(case, flags=0, c_layout="row", out=None):
    import torch
    ll = _ll()
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    if out is None:
        if c_layout == "row":
            C = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
        else:
            C = torch.full((case.N, case.M), float("nan"), dtype=dt, device="cuda").t()
    else:
        C = out
    ll.gemm(A, B, out=C, flags=flags)
    torch.cuda.synchronize()
    return C


def _full_check(case, flags=0, c_layout="row"):
    C = _run(case, flags, c_layout)
    ref, S = oracle.gemm_case(case)
    acceptance.assert_close(to_f64(C), ref, S, case.out_dtype,
                            f"{case.name} M={case.M} N={case.N} K={case.K} flags={flags}")
    return C, ref


def test_gemm_256_fp32_out_full():
    case = synth.gemm_workload("gemm_256")
    _full_check(case)


SHAPES = [(1, 1, 1), (7, 9, 13), (33, 65, 129), (128, 128, 64), (200, 136, 72), (257, 263, 300),
          (64, 520, 8), (300, 8, 1000), (130, 1030, 520)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_small_shapes_every_layout(M, N, K, la, lb):
    seed = M * 1000003 + N * 1009 + K
    c = synth.gemm_case(M, N, K, seed=seed, b_col_major=(lb == "col"), out_dtype="f32")
    if la == "col":  # re-describe A column-major: buffer is [K][M]
        c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=seed, tensor=5)
        c.sam, c.sak = 1, M
    _full_check(c)
    c.out_dtype = "bf16"
    _full_check(c)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (257, 263, 300), (520, 264, 1992)])
def test_integer_inputs_bit_exact(M, N, K):
    c = synth.gemm_case(M, N, K, dist=("int", -4, 4), seed=M + N + K)
    C = _run(c)
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(to_f64(C), ref)


def test_bf16_epilogue_rounds_to_nearest_even():
    # Integer-valued results up to ~2^12 are exact in fp32 and mostly need rounding to 8 bits.
    c = synth.gemm_case(256, 256, 256, dist=("int", -4, 4), seed=99, out_dtype="bf16")
    C = _run(c)
    ref, _ = oracle.gemm_case(c)
    want = synth.f32_to_bf16_rne(ref.astype(np.float32))
    import torch
    got = C.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_k_zero_and_empty():
    import torch
    ll = _ll()
    A = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((0, 7), dtype=torch.bfloat16, device="cuda")
    C = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    ll.gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    A = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((16, 7), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((0, 7), dtype=torch.float32, device="cuda")
    ll.gemm(A, B, out=C)
    torch.cuda.synchronize()


@pytest.mark.parametrize("flags", [0, 0x1, 0x2, 0x3, 0x4, 0x8])
def test_modes_agree(flags):
    c = synth.gemm_case(520, 1032, 264, dist=("int", -4, 4), seed=5)
    C = _run(c, flags=flags)
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(to_f64(C), ref)
    c2 = synth.gemm_case(333, 555, 777, seed=6, dist=("normal", 0, 1.0), out_dtype="bf16")
    _full_check(c2, flags=flags)


def test_column_major_c():
    c = synth.gemm_case(200, 300, 136, seed=8)
    _full_check(c, c_layout="col")


def test_misaligned_operand_is_rejected_without_pack():
    import torch
    ll = _ll()
    base = torch.zeros(64 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    A = base[1:].view(64, 64)
    B = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ll.LLError) as e:
        ll.gemm(A, B, out=C)
    assert e.value.status == ll.LL_ERR_INVALID_ARG
    ll.gemm(A, B, out=C, flags=ll.LL_FLAG_PACK_A)
    torch.cuda.synchronize()


@pytest.mark.parametrize("offset", [0, 1, 2, 3])
@pytest.mark.parametrize("ldb", [300, 301])
@pytest.mark.parametrize("a_col", [False, True])
def test_packed_b_from_any_2_byte_offset(offset, ldb, a_col):
    """Column-major B packed from a view that starts at any 2-byte offset:
    the packs read a row's interior as aligned words and must shift by the
    view's own address, not by the element index.  Beside a K-contiguous A
    the copy stays K-contiguous (the row copy); beside an M-contiguous A it
    is transposed N-contiguous (the LDS transpose)."""
    import torch
    ll = _ll()
    M, N, K = 136, 70, 290
    seed = 91 + offset * 7 + ldb + 50 * a_col
    c = synth.gemm_case(M, N, K, seed=seed, b_col_major=True, ldb=ldb, out_dtype="f32")
    if a_col:
        c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=seed, tensor=5)
        c.sam, c.sak = 1, M
    B_bits = np.concatenate([np.zeros(offset, dtype=np.uint16), c.B])
    base = torch.from_numpy(B_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    B = torch.as_strided(base, (K, N), (1, ldb), offset)
    A, _ = gemm_operands(c)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ll.gemm(A, B, out=C, flags=ll.LL_FLAG_PACK_B)
    torch.cuda.synchronize()
    d = ll.plan_for(A, B, C, ll.LL_FLAG_PACK_B).describe()
    assert ("B:N-major" if a_col else "B:K-major") in d and "packB=1" in d, d
    assert ("packA=0" in d) == a_col, d  # K = 290: a K-contiguous A is packed too
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C), ref, S, "f32", f"packed B offset {offset} ldb {ldb}")


def _sampled_check(case, n=4096, strip_rows=64, seed=1, flags=0):
    """Full-size parity: n seeded entries (with the corners and the last tile
    row and column), one seeded entry in every output tile of the plan's tile
    grid, a seeded strip of strip_rows rows, and the first and last rows, each
    against the oracle."""
    import torch
    ll = _ll()
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    C = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    ll.gemm(A, B, out=C, flags=flags)
    torch.cuda.synchronize()
    tile = plan_tile(ll.plan_for(A, B, C, flags).describe())
    del A, B
    got = to_f64(C)
    del C
    rows, cols = sample_indices(case.M, case.N, n, seed, tile=tile)
    tr, tc = per_tile_indices(case.M, case.N, tile, seed + 1)
    rows, cols = np.concatenate([rows, tr]), np.concatenate([cols, tc])
    ref, S = oracle.gemm_case_entries(case, rows, cols)
    acceptance.assert_close(got[rows, cols], ref, S, case.out_dtype, f"{case.name} samples (tile {tile})")
    for r0, nr in strip_starts(case.M, strip_rows, seed + 2):
        ref, S = oracle.gemm_case(case, rows=(r0, nr))
        acceptance.assert_close(got[r0:r0 + nr], ref, S, case.out_dtype, f"{case.name} rows {r0}..{r0 + nr - 1}")
    return got


def test_gemm_4096_bf16_out():
    _sampled_check(synth.gemm_workload("gemm_4096"))


@pytest.mark.parametrize("name", ["ffn_up", "ffn_down"])
def test_ffn_shapes(name):
    _sampled_check(synth.gemm_workload(name))


@pytest.mark.parametrize("name,layout", [("ffn_up", "b_col_major"), ("ffn_down", "a_col_major")])
def test_ffn_shapes_other_layouts(name, layout):
    """The FFN shapes with B K-contiguous (the forward X W^T; ffn_up also
    prefetches its wide B) and with A M-contiguous (a weight gradient's
    layout): the hand-ordered kind's variants with the round barrier, one
    entry in every tile, random entries and row strips against the oracle."""
    import torch
    ll = _ll()
    M, N, K, kw = synth.GEMM_WORKLOADS[name]
    case = synth.gemm_case(M, N, K, name=f"{name}_{layout}", **dict(kw, **{layout: True}))
    _sampled_check(case, n=2048, strip_rows=16)
    A, B = gemm_operands(case)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    d = ll.plan_for(A, B, C).describe()
    want = "A:K-major,B:K-major" if layout == "b_col_major" else "A:M-major,B:N-major"
    assert "kernel=KIND_SQ4_HO " in d and want in d and "round_sync=1" in d and "packA=0 packB=0" in d, d
    if name == "ffn_up":
        assert "prefetch_b=1" in d, d


def test_descriptor_rebase_past_1gib():
    """A row-major B whose k-range per work item spans more than 1 GiB (the
    loader re-opens its buffer descriptor at the current slice once the
    running offset passes 2^30): 2048 x 28672 x 24576, B 1.41 GB, no K split."""
    c = synth.gemm_case(2048, 28672, 24576, dist=("normal", 0.0, 1.0), b_dist=("normal", 0.0, 0.02),
                        seed=12, out_dtype="bf16", name="rebase_1gib")
    slice_bytes = 64 * c.sbk * 2
    assert slice_bytes * (c.K // 64) > 1 << 30
    import torch
    A, B = gemm_operands(c)
    d = _ll().plan_for(A, B, torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")).describe()
    del A, B
    assert "splitk=1 " in d and "packB=0" in d and "B:N-major" in d, d
    _sampled_check(c, strip_rows=16)


@pytest.mark.parametrize("M,N,K,kind", [(384, 520, 1017, None), (2048, 2048, 4095, "KIND_SQ8_LW4"),
                                        (2048, 2048, 4095, "KIND_SQ4_HO"), (1000, 1032, 2043, "KIND_SQ4_HO"),
                                        (1000, 1032, 2043, "KIND_WIDE_PC"), (520, 1032, 1982, "KIND_TALL_PC"),
                                        (1000, 1032, 2044, "KIND_T192_PC"), (520, 264, 1021, "KIND_WIDE_COOP")])
def test_packed_a_with_direct_b_reads_no_row_past_k(M, N, K, kind, monkeypatch):
    """K = 57..63 mod 64 with a row-major A (packed: K is not a multiple of 8, its
    copy carries zero columns up to K rounded to 8, a whole number of 64-deep
    slices) and a row-major B read in place: B is a view of the first K rows of a
    buffer whose later rows are NaN.  The last slice must take the masked load
    path, since B holds only K rows; any read of a row past K shows as NaN."""
    import torch
    ll = _ll()
    assert K % 64 >= 57 and K % 8 != 0
    c = synth.gemm_case(M, N, K, seed=K + M, out_dtype="f32", name="k_tail")
    A, _ = gemm_operands(c)
    Bfull = torch.full((K + 16, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Bfull[:K] = gemm_operands(c)[1]
    B = Bfull[:K]
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ll._plans.clear()
    if kind:
        monkeypatch.setenv("LL_GEMM_KIND", kind)
    try:
        ll.gemm(A, B, out=C)
        torch.cuda.synchronize()
        desc = ll.plan_for(A, B, C).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()
    assert "packA=1" in desc and "packB=0" in desc, desc
    if kind:
        assert f"kernel={kind} " in desc, desc
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C), ref, S, "f32", f"{M}x{N}x{K} {desc}")


def test_edge_shape_column_major_b():
    _sampled_check(synth.gemm_workload("edge"))


def test_edge_shape_integer_exact_samples():
    M, N, K, kw = synth.GEMM_WORKLOADS["edge"]
    kw = dict(kw, dist=("int", -4, 4))
    c = synth.gemm_case(M, N, K, name="edge_int", **kw)
    got = to_f64(_run(c))
    rows, cols = sample_indices(M, N, 4096, 3)
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(got[rows, cols], ref)


def test_skinny_split_k():
    import torch
    ll = _ll()
    c = synth.gemm_workload("skinny_splitk")
    A, B = gemm_operands(c)
    assert "splitk=1 " not in ll.plan_for(A, B, torch.empty((c.M, c.N), device="cuda")).describe()
    got = _sampled_check(c)
    again = to_f64(_run(c))
    assert np.array_equal(got, again), "split-K result must be run-to-run deterministic"


def test_skinny_split_k_integer_exact():
    M, N, K, kw = synth.GEMM_WORKLOADS["skinny_splitk"]
    kw = dict(kw, dist=("int", -1, 1))
    c = synth.gemm_case(M, N, K, name="skinny_int", **kw)
    got = to_f64(_run(c))
    rows, cols = sample_indices(M, N, 2048, 4)
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(got[rows, cols], ref)


# ---------------------------------------------------------------------------
# fp16 operands (same data path, v_mfma_f32_32x32x16_f16)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(7, 9, 13), (200, 136, 72), (257, 263, 300), (130, 1030, 520)])
@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_f16_small_shapes_every_layout(M, N, K, la, lb):
    seed = M * 7919 + N * 31 + K
    c = synth.gemm_case(M, N, K, seed=seed, b_col_major=(lb == "col"), out_dtype="f32", in_dtype="f16")
    if la == "col":
        c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=seed, tensor=5, fmt="f16")
        c.sam, c.sak = 1, M
    for out in ("f32", "f16", "bf16"):
        c.out_dtype = out
        _full_check(c)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (257, 263, 300)])
def test_f16_integer_inputs_bit_exact(M, N, K):
    c = synth.gemm_case(M, N, K, dist=("int", -4, 4), seed=M + N + K + 7, in_dtype="f16")
    C = _run(c)
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(to_f64(C), ref)


def test_f16_epilogue_rounds_to_nearest_even():
    # integer-valued sums, exact in fp32, rounded once to fp16
    c = synth.gemm_case(256, 256, 256, dist=("int", -8, 8), seed=98, out_dtype="f16", in_dtype="f16")
    C = _run(c)
    ref, _ = oracle.gemm_case(c)
    want = synth.f32_to_f16_rne(ref.astype(np.float32))
    import torch
    got = C.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_split_k_and_k_zero():
    import torch
    ll = _ll()
    c = synth.gemm_case(128, 1024, 8192, seed=97, out_dtype="f16", in_dtype="f16")
    _full_check(c)
    A = torch.zeros((5, 0), dtype=torch.float16, device="cuda")
    B = torch.zeros((0, 7), dtype=torch.float16, device="cuda")
    C = torch.full((5, 7), 3.0, dtype=torch.float16, device="cuda")
    ll.gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)


def test_mixed_operand_types_rejected():
    import torch
    ll = _ll()
    A = torch.zeros((8, 8), dtype=torch.float16, device="cuda")
    B = torch.zeros((8, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ll.LLError):
        ll.gemm(A, B)


def test_gemm_4096_f16_sampled():
    _sampled_check(synth.gemm_workload("gemm_4096_f16"))


def test_gemm_4096_nt_sampled():
    # B K-contiguous (C = X W^T): the hand-ordered kind's variant for such a B, in place
    _sampled_check(synth.gemm_workload("gemm_4096_nt"))


def test_gemm_4096_tn_sampled():
    # A M-contiguous (C = X^T Y): the hand-ordered kind's variant for such an A, in place
    _sampled_check(synth.gemm_workload("gemm_4096_tn"))
