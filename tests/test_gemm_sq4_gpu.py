"""The hand-ordered 256x256 kind (four waves of 128x128, KIND_SQ4_HO) forced on
shapes of every kind of edge, against the fp64 oracle: ragged M and N, one,
two, three and many 64-deep slices, split K, bf16 and fp16 operands, every
output type, packed operands, integer inputs bit for bit, and full size."""
import re

import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_operands, per_tile_indices, plan_tile, sample_indices, strip_starts, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu
KIND = "KIND_SQ4_HO"


def _run(case, monkeypatch, flags=0):
    import torch
    import recsys_linear_layers_amd as ll
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    C = torch.full((case.M, case.N), float("nan"), dtype=dt, device="cuda")
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    try:
        ll.gemm(A, B, out=C, flags=flags)
        torch.cuda.synchronize()
        d = ll.plan_for(A, B, C, flags).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()
    assert f"kernel={KIND} " in d, d
    return to_f64(C), d


SHAPES = [(256, 256, 64), (256, 256, 128), (256, 256, 192), (256, 512, 1024), (300, 520, 640),
          (1000, 1032, 2048), (513, 264, 320), (8, 8, 64), (40, 24, 448), (1536, 1280, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_shapes(M, N, K, out, monkeypatch):
    c = synth.gemm_case(M, N, K, seed=M * 7 + N * 3 + K, out_dtype=out, dist=("normal", 0.0, 1.0))
    got, d = _run(c, monkeypatch)
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, out, f"{M}x{N}x{K} {d}")


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (520, 264, 1024), (300, 1032, 640)])
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_f16_operands(M, N, K, out, monkeypatch):
    c = synth.gemm_case(M, N, K, seed=M + N + K + 5, out_dtype=out, in_dtype="f16")
    got, d = _run(c, monkeypatch)
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, out, f"f16 {M}x{N}x{K} {d}")


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (520, 776, 1984), (128, 4096, 16384)])
def test_integer_inputs_bit_exact(M, N, K, monkeypatch):
    # the last shape splits K (16 tiles on 256 CUs): partials plus the ordered reduce
    c = synth.gemm_case(M, N, K, dist=("int", -4, 4), seed=M + N + K + 9)
    got, d = _run(c, monkeypatch)
    ref, _ = oracle.gemm_case(c)
    assert np.array_equal(got, ref), d


def test_packed_a(monkeypatch):
    # a column-major A is packed K-contiguous; B stays N-contiguous
    M, N, K = 300, 520, 640
    c = synth.gemm_case(M, N, K, seed=77, out_dtype="f32")
    c.A = synth.bf16_tensor(M * K, "uniform", -1.0, 1.0, seed=77, tensor=5)
    c.sam, c.sak = 1, M
    got, d = _run(c, monkeypatch)
    assert "packA=1" in d
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, "f32", d)


@pytest.mark.parametrize("M,N,K,lda", [(520, 264, 1091, 1093), (300, 776, 200, 201), (256, 256, 72, 73)])
def test_k_tail_with_packed_a(M, N, K, lda, monkeypatch):
    """K not a multiple of 64 with an A whose odd row stride makes the plan
    pack it (zero columns up to K rounded to 64): the last slice reads B rows
    past K as zeros through the descriptor range."""
    c = synth.gemm_case(M, N, K, seed=M + N + K + 11, lda=lda, out_dtype="bf16", dist=("normal", 0.0, 1.0))
    got, d = _run(c, monkeypatch)
    assert "packA=1" in d, d
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, "bf16", f"k tail {M}x{N}x{K} lda={lda} {d}")


def test_refused_where_it_does_not_apply(monkeypatch):
    import torch
    import recsys_linear_layers_amd as ll
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    try:
        A = torch.zeros((256, 200), dtype=torch.bfloat16, device="cuda")  # K not a multiple of 64
        B = torch.zeros((200, 256), dtype=torch.bfloat16, device="cuda")
        C = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
        with pytest.raises(ll.LLError) as e:
            ll.GemmPlan(ll.gemm_desc_for(A, B, C), A.device)
        assert e.value.status == ll.LL_ERR_UNSUPPORTED
        # K = 200 with A packed (row stride 201) but a K-contiguous B read in
        # place: its rows past K would meet A's zero columns with the next
        # row's values
        A2 = torch.zeros((256, 201), dtype=torch.bfloat16, device="cuda")[:, :200]
        Bc = torch.zeros((256, 200), dtype=torch.bfloat16, device="cuda").t()
        with pytest.raises(ll.LLError) as e:
            ll.GemmPlan(ll.gemm_desc_for(A2, Bc, C), A2.device)
        assert e.value.status == ll.LL_ERR_UNSUPPORTED
        # a K-contiguous B with K a multiple of 64 is taken
        Bk = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda").t()
        A3 = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
        assert "B:K-major" in ll.GemmPlan(ll.gemm_desc_for(A3, Bk, C), A3.device).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)


def _describe(M, N, K, a_col=False, b_col=False, in_t=0, c_t=0, flags=0, epilogue=0):
    import recsys_linear_layers_amd as ll
    sam, sak = (1, M) if a_col else (K, 1)
    sbk, sbn = (1, K) if b_col else (N, 1)
    h = ll.gemm_plan_create(ll.GemmDesc(M, N, K, sam, sak, sbk, sbn, N, 1, in_t, in_t, c_t, flags, epilogue))
    try:
        return ll.gemm_plan_describe(h)
    finally:
        ll.gemm_plan_destroy(h)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (16384, 28672, 8192), (16384, 8192, 28672),
                                   (8192, 8192, 8192), (4096, 4096, 16384), (4000, 4000, 640)])
def test_selected_on_square_and_ffn_shapes(M, N, K):
    assert f"kernel={KIND} " in _describe(M, N, K)


@pytest.mark.parametrize("M,N,K,want", [(4096, 4096, 4096, True), (16384, 28672, 8192, True),
                                     (16384, 8192, 28672, True), (8192, 2048, 8192, True), (2048, 8192, 8192, True),
                                     (3072, 3072, 3072, False), (4096, 1024, 2048, False), (4096, 2560, 1024, False)])
def test_k_contiguous_b_selected_in_place(M, N, K, want):
    """C = X W^T (B K-contiguous, W stored [N][K]): the hand-ordered kind takes
    B in place, its tiles laid out and read like A's, under the same area rule
    as for an N-contiguous B (3072^3 and 4096 x 2560: 192x256 tiles; 64 tiles
    of 256x256: split K).  Asked for producer/consumer kernels, it stays out."""
    import recsys_linear_layers_amd as ll
    d = _describe(M, N, K, b_col=True)
    assert (f"kernel={KIND} " in d) == want, d
    assert "packB=0" in d and "B:K-major" in d, d
    assert (f"kernel={KIND} " in _describe(M, N, K)) == want
    d = _describe(M, N, K, b_col=True, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    assert f"kernel={KIND} " not in d, d


def test_k_contiguous_b_integer_exact():
    """The hand-ordered kind with B K-contiguous against the producer/consumer
    kind on the same B: integer inputs make both exact, so the bits agree, and
    sampled entries match the oracle."""
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.gemm_case(4096, 4096, 1024, dist=("int", -4, 4), seed=341, out_dtype="f32", b_col_major=True)
    A, B = gemm_operands(c)
    C1 = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ll._plans.clear()
    ll.gemm(A, B, out=C1)
    ll.gemm(A, B, out=C2, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    torch.cuda.synchronize()
    d1 = ll.plan_for(A, B, C1).describe()
    d2 = ll.plan_for(A, B, C2, ll.LL_FLAG_PRODUCER_CONSUMER).describe()
    ll._plans.clear()
    assert f"kernel={KIND} " in d1 and "B:K-major" in d1 and "packB=0" in d1, d1
    assert f"kernel={KIND} " not in d2, d2
    g1, g2 = to_f64(C1), to_f64(C2)
    assert np.array_equal(g1, g2), (d1, d2)
    rows, cols = sample_indices(c.M, c.N, 2048, 342, tile=plan_tile(d1))
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(g1[rows, cols], ref)


@pytest.mark.parametrize("b_col", [False, True])
def test_m_contiguous_a_selected_in_place(b_col):
    """C = X^T Y (A M-contiguous, a layer's weight gradient): the hand-ordered
    kind takes A in place, its tiles laid out and read like an N-contiguous
    B's, B either way; also with K not a multiple of 64 when B is
    N-contiguous (both operands then read zeros past K)."""
    import recsys_linear_layers_amd as ll
    lay = "A:M-major,B:K-major" if b_col else "A:M-major,B:N-major"
    for M, N, K in [(4096, 4096, 4096), (16384, 8192, 8192), (8192, 2048, 8192)]:
        d = _describe(M, N, K, a_col=True, b_col=b_col)
        assert f"kernel={KIND} " in d and lay in d and "packA=0" in d and "packB=0" in d, d
    d = _describe(4096, 4096, 4104, a_col=True, b_col=b_col)
    assert (f"kernel={KIND} " in d) == (not b_col), d     # a K-contiguous B in place needs K % 64 == 0
    d = _describe(4096, 4096, 4096, a_col=True, b_col=b_col, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    assert f"kernel={KIND} " not in d, d


AM_SHAPES = [(256, 256, 64), (256, 256, 192), (1000, 1032, 2048), (8, 8, 64), (40, 24, 448), (1536, 1280, 512),
             (264, 520, 200), (1000, 1032, 130)]


def _am_case(M, N, K, seed, out, b_col, in_dtype="bf16", dist=("normal", 0.0, 1.0)):
    c = synth.gemm_case(M, N, K, seed=seed, out_dtype=out, in_dtype=in_dtype, dist=dist, b_col_major=b_col)
    c.A = synth.bf16_tensor(M * K, dist[0], dist[1], dist[2], seed=seed, tensor=5, fmt=in_dtype)
    c.sam, c.sak = 1, M
    return c


@pytest.mark.parametrize("M,N,K", AM_SHAPES)
@pytest.mark.parametrize("b_col", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_shapes_a_m_contiguous(M, N, K, b_col, out, monkeypatch):
    """The variants for an M-contiguous A forced on ragged M and N, one to many
    slices, B either way; with K not a multiple of 64 the M-contiguous A reads
    zeros past K in place, and a K-contiguous B is packed."""
    import recsys_linear_layers_amd as ll
    c = _am_case(M, N, K, M * 3 + N * 5 + K + b_col, out, b_col)
    flags = ll.LL_FLAG_PACK_B if (b_col and K % 64) else 0   # packed N-contiguous beside an M-contiguous A
    got, d = _run(c, monkeypatch, flags)
    assert ("A:M-major,B:K-major" if b_col and not flags else "A:M-major,B:N-major") in d and "packA=0" in d, d
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, out, f"A M-contiguous {M}x{N}x{K} {d}")


@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("out,in_dtype", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16")])
def test_a_m_contiguous_epilogue_and_f16(act, out, in_dtype, monkeypatch):
    """Bias + activation, fp16 operands and every C type with A M-contiguous,
    304 x 1032 x 640."""
    import torch
    M, N, K = 304, 1032, 640
    c = _am_case(M, N, K, 351, out, False, in_dtype=in_dtype)
    A, B = gemm_operands(c)
    bias = torch.from_numpy(np.random.default_rng(352).standard_normal(N).astype(np.float32)).cuda()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    d = _run_into(A, B, C, monkeypatch, bias, act)
    assert "A:M-major" in d, d
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(to_f64(C), ref, S, out, f"A M-contiguous {out} act={act} {d}", act=act)


@pytest.mark.parametrize("b_col", [False, True])
def test_m_contiguous_a_integer_exact(b_col):
    """A M-contiguous in the hand-ordered kind (chosen by the plan) against the
    producer/consumer kind on the same operands: integer inputs make both
    exact, so the bits agree; sampled entries match the oracle.  4352 x 4160
    x 4096: the K-split last round (tail=33x4) runs too."""
    import torch
    import recsys_linear_layers_amd as ll
    c = _am_case(4352, 4160, 4096, 353 + b_col, "f32", b_col, dist=("int", -3, 3))
    A, B = gemm_operands(c)
    C1 = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
    ll._plans.clear()
    ll.gemm(A, B, out=C1)
    ll.gemm(A, B, out=C2, flags=ll.LL_FLAG_PRODUCER_CONSUMER)
    torch.cuda.synchronize()
    d1 = ll.plan_for(A, B, C1).describe()
    d2 = ll.plan_for(A, B, C2, ll.LL_FLAG_PRODUCER_CONSUMER).describe()
    ll._plans.clear()
    assert f"kernel={KIND} " in d1 and "A:M-major" in d1 and " tail=33x4" in d1, d1
    assert f"kernel={KIND} " not in d2, d2
    g1, g2 = to_f64(C1), to_f64(C2)
    assert np.array_equal(g1, g2), (d1, d2)
    rows, cols = sample_indices(c.M, c.N, 2048, 354, tile=256)
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(g1[rows, cols], ref)


BK_SHAPES = [(256, 256, 64), (256, 256, 192), (300, 520, 640), (1000, 1032, 2048), (513, 264, 320), (8, 8, 64),
             (40, 24, 448), (1536, 1280, 512)]


@pytest.mark.parametrize("M,N,K", BK_SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_shapes_b_k_contiguous(M, N, K, out, monkeypatch):
    """The variant for a K-contiguous B forced on ragged M and N, one to many
    slices, both output types."""
    c = synth.gemm_case(M, N, K, seed=M * 5 + N * 7 + K, out_dtype=out, dist=("normal", 0.0, 1.0), b_col_major=True)
    got, d = _run(c, monkeypatch)
    assert "B:K-major" in d and "packB=0" in d, d
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(got, ref, S, out, f"B K-contiguous {M}x{N}x{K} {d}")


@pytest.mark.parametrize("act", [None, "gelu"])
@pytest.mark.parametrize("out,in_dtype", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16")])
def test_b_k_contiguous_epilogue_and_f16(act, out, in_dtype, monkeypatch):
    """Bias + activation, fp16 operands and every C type with B K-contiguous,
    300 x 1032 x 640 (ragged M, several tiles)."""
    import torch
    import recsys_linear_layers_amd as ll
    M, N, K = 300, 1032, 640
    c = synth.gemm_case(M, N, K, seed=343, out_dtype=out, in_dtype=in_dtype, dist=("normal", 0.0, 1.0),
                        b_col_major=True)
    A, B = gemm_operands(c)
    bias = torch.from_numpy(np.random.default_rng(344).standard_normal(N).astype(np.float32)).cuda()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    d = _run_into(A, B, C, monkeypatch, bias, act)
    assert "B:K-major" in d, d
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(to_f64(C), ref, S, out, f"B K-contiguous {out} act={act} {d}", act=act)


def test_b_k_contiguous_tail_split_and_round_barrier(monkeypatch):
    """The K-split last round (4300 x 4100 x 4096: 33 tiles split 4 ways) and,
    forced on, the round barrier with B K-contiguous: the same bits as without
    them on integer inputs, and the oracle on sampled entries."""
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.gemm_case(4300, 4100, 4096, dist=("int", -3, 3), seed=345, out_dtype="f32", b_col_major=True)
    A, B = gemm_operands(c)
    outs = []
    for tail, sync in (("1", "0"), ("0", "0"), ("1", "1")):
        monkeypatch.setenv("LL_GEMM_TAIL_SPLIT", tail)
        monkeypatch.setenv("LL_GEMM_ROUND_SYNC", sync)
        C = torch.full((c.M, c.N), float("nan"), dtype=torch.float32, device="cuda")
        d = _run_into(A, B, C, monkeypatch)
        outs.append((to_f64(C), d))
    monkeypatch.delenv("LL_GEMM_TAIL_SPLIT", raising=False)
    monkeypatch.delenv("LL_GEMM_ROUND_SYNC", raising=False)
    assert " tail=33x4" in outs[0][1] and " tail=0x1" in outs[1][1], [d for _, d in outs]
    assert "B:K-major" in outs[0][1]
    for g, d in outs[1:]:
        assert np.array_equal(outs[0][0], g), d
    rows, cols = sample_indices(c.M, c.N, 2048, 346, tile=256)
    ref, _ = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(outs[0][0][rows, cols], ref)


@pytest.mark.parametrize("M,N,K,b_col,want", [
    (8448, 8448, 4096, False, True),    # 5 passes of 256x256 against 9 of 256x128: 1.11x the area
    (12288, 4608, 8192, False, True),   # 4 against 7 of 128x256: 1.14x
    (8191, 5003, 4099, True, True),     # the edge shape, both operands packed: 3 against 5, 1.2x
    (4608, 4608, 4096, False, True),    # 1 + 1/3 (last round split 3 ways) against 3 of 256x128: 0.89x
    (6144, 6144, 4096, False, True),    # 2 + 1/4 against 3 of 192x256: 1.0x
    (4352, 4352, 1024, False, False),   # 2 (16 slices: no split) against 3 of 256x128: 1.33x
])
def test_selected_up_to_a_quarter_more_area(M, N, K, b_col, want):
    """The hand-ordered kind runs ~1.3x as fast per pass and tile area as the
    other kinds, so it is chosen while it needs at most 1.25x their passes
    times tile area, a last round it splits s ways along K counting 1/s."""
    assert (f"kernel={KIND} " in _describe(M, N, K, b_col=b_col)) == want


def test_selection_conditions():
    import recsys_linear_layers_amd as ll
    assert f"kernel={KIND} " in _describe(4096, 4096, 4096, in_t=ll.LL_F16, c_t=ll.LL_F16)
    assert f"kernel={KIND} " in _describe(4096, 4096, 4096, c_t=ll.LL_F32)
    assert f"kernel={KIND} " in _describe(4096, 4096, 4096, epilogue=ll.LL_EPI_GELU)
    assert f"kernel={KIND} " in _describe(4096, 4096, 4096, epilogue=ll.LL_EPI_BIAS | ll.LL_EPI_SILU)
    # (a K-contiguous B or an M-contiguous A: the tests of those variants)
    for kw in (dict(flags=ll.LL_FLAG_PRODUCER_CONSUMER), dict(flags=ll.LL_FLAG_COOPERATIVE)):
        assert f"kernel={KIND} " not in _describe(4096, 4096, 4096, **kw), kw
    assert f"kernel={KIND} " not in _describe(4096, 4096, 4104)        # K % 64 != 0
    assert f"kernel={KIND} " not in _describe(2048, 4096, 8192)        # 128 tiles would split K
    assert f"kernel={KIND} " not in _describe(128, 8192, 65536)        # skinny


@pytest.mark.parametrize("act", [None, "relu", "gelu", "silu"])
@pytest.mark.parametrize("M,N,K,out", [(300, 520, 640, "f32"), (513, 264, 320, "bf16"), (256, 256, 64, "f32"),
                                       (128, 4096, 16384, "bf16")])
def test_fused_bias_activation(act, M, N, K, out, monkeypatch):
    """Per-column bias and ReLU / GELU / SiLU on the fp32 sums before the store;
    the last shape splits K (the ordered reduce applies the epilogue)."""
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.gemm_case(M, N, K, seed=M + 2 * N + 3 * K, out_dtype=out, dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    bias = torch.from_numpy(np.random.default_rng(M + N).standard_normal(N).astype(np.float32)).cuda()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    try:
        ll.gemm(A, B, out=C, bias=bias, act=act)
        torch.cuda.synchronize()
        d = ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.ACTIVATIONS[act]).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()
    assert f"kernel={KIND} " in d, d
    ref, S = oracle.gemm_case(c)
    ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(to_f64(C), ref, S, out, f"{M}x{N}x{K} bias+{act} {d}", act=act)


@pytest.mark.parametrize("name", ["gemm_4096", "ffn_up"])
def test_full_size_sampled(name, monkeypatch):
    c = synth.gemm_workload(name)
    got, d = _run(c, monkeypatch)
    tile = plan_tile(d)
    rows, cols = sample_indices(c.M, c.N, 4096, 5, tile=tile)
    tr, tc = per_tile_indices(c.M, c.N, tile, 6)
    rows, cols = np.concatenate([rows, tr]), np.concatenate([cols, tc])
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    acceptance.assert_close(got[rows, cols], ref, S, c.out_dtype, f"{name} samples {d}")
    for r0, nr in strip_starts(c.M, 64, 7):
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        acceptance.assert_close(got[r0:r0 + nr], ref, S, c.out_dtype, f"{name} rows {r0}.. {d}")


def _run_into(A, B, C, monkeypatch, bias=None, act=None):
    import torch
    import recsys_linear_layers_amd as ll
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    try:
        ll.gemm(A, B, out=C, bias=bias, act=act)
        torch.cuda.synchronize()
        ep = (ll.LL_EPI_BIAS if bias is not None else 0) | ll.ACTIVATIONS[act]
        d = ll.plan_for(A, B, C, 0, ep).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()
    assert f"kernel={KIND} " in d, d
    return d


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("act", [None, "gelu"])
def test_staged_epilogue_matches_direct_stores(out, act, monkeypatch):
    """Whole tiles of a 16-bit C whose rows are 16-byte aligned leave through
    an LDS image with 16-byte stores; with a row stride that is not a multiple
    of 8 elements every tile takes the direct 4-byte stores.  Both give the
    same bits.  4600 x 4352: 18 x 17 = 306 tiles on 256 workgroups (a second
    work item for 50 of them, after the barrier that guards the image), the
    last tile row ragged (direct stores beside staged tiles); checked against
    the oracle in full."""
    import torch
    in_dtype = "f16" if out == "f16" else "bf16"
    M, N, K = 4600, 4352, 128
    c = synth.gemm_case(M, N, K, seed=91 + (act is None), out_dtype=out, in_dtype=in_dtype,
                        dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[out]
    bias = None
    if act:
        bias = torch.from_numpy(np.random.default_rng(92).standard_normal(N).astype(np.float32)).cuda()
    C1 = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    big = torch.full((M, N + 4), float("nan"), dtype=dt, device="cuda")
    C2 = big[:, :N]
    d1 = _run_into(A, B, C1, monkeypatch, bias, act)
    d2 = _run_into(A, B, C2, monkeypatch, bias, act)
    g1, g2 = to_f64(C1), to_f64(C2)
    assert np.array_equal(g1, g2), (d1, d2)
    assert torch.isnan(big[:, N:].float()).all()  # the padding columns are untouched
    ref, S = oracle.gemm_case(c)
    if act:
        ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(g1, ref, S, out, f"staged {M}x{N}x{K} {out} act={act} {d1}", act=act)


@pytest.mark.parametrize("act", [None, "relu", "gelu", "silu"])
def test_f32_whole_tile_stores_match_general_path(act, monkeypatch):
    """Whole tiles of an fp32 C with unit column stride take one store per
    element from a per-lane row pointer, also for a row stride that is odd
    (4-byte aligned rows only); a column-major C and the ragged last tile row
    take the general per-element path.  All give the same bits, the padding
    columns stay untouched, and the result matches the oracle in full.
    4600 x 4352 x 128: 306 tiles on 256 workgroups."""
    import torch
    M, N, K = 4600, 4352, 128
    c = synth.gemm_case(M, N, K, seed=97 + len(str(act)), out_dtype="f32", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    bias = None
    if act:
        bias = torch.from_numpy(np.random.default_rng(98).standard_normal(N).astype(np.float32)).cuda()
    C1 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    big = torch.full((M, N + 3), float("nan"), dtype=torch.float32, device="cuda")
    C2 = big[:, :N]
    C3 = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda").t()
    ds = [_run_into(A, B, C, monkeypatch, bias, act) for C in (C1, C2, C3)]
    g1, g2, g3 = to_f64(C1), to_f64(C2), to_f64(C3)
    assert np.array_equal(g1, g2), ds
    assert np.array_equal(g1, g3), ds
    assert torch.isnan(big[:, N:]).all()
    ref, S = oracle.gemm_case(c)
    if act:
        ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
    acceptance.assert_close(g1, ref, S, "f32", f"f32 whole tiles {M}x{N}x{K} act={act} {ds[0]}", act=act)


def test_staged_epilogue_needs_16_byte_aligned_c(monkeypatch):
    """A C that starts 8 bytes into an allocation (rows 16-byte aligned apart
    from that) takes the direct stores and matches an aligned C."""
    import torch
    M, N, K = 512, 768, 192
    c = synth.gemm_case(M, N, K, seed=93, out_dtype="bf16", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    C1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    flat = torch.full((M * N + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    C2 = flat[4:4 + M * N].view(M, N)
    assert C2.data_ptr() % 16 == 8
    _run_into(A, B, C1, monkeypatch)
    _run_into(A, B, C2, monkeypatch)
    assert np.array_equal(to_f64(C1), to_f64(C2))
    ref, S = oracle.gemm_case(c)
    acceptance.assert_close(to_f64(C1), ref, S, "bf16", "aligned C")


def test_round_barrier_selection(monkeypatch):
    """Plans of the hand-ordered kind with 8 rounds of tiles or more, each of
    K >= 8192 (128 slices), keep
    each XCD's workgroups a round apart at most (round_sync=1), with their
    counters in the workspace; fewer rounds and other kinds do not, and the
    override turns it on from two rounds or off."""
    import recsys_linear_layers_amd as ll
    for M, N, K in [(16384, 28672, 8192), (16384, 8192, 28672), (16384, 8192, 8192)]:   # 28, 8, 8 rounds
        d = _describe(M, N, K)
        assert f"kernel={KIND} " in d and "round_sync=1" in d, d
        assert int(d.split(" ws=")[1].split()[0]) >= 1024, d
    for M, N, K in [(4096, 4096, 4096), (8192, 8192, 8192), (16384, 16384, 4096), (4096, 8192, 8192)]:
        d = _describe(M, N, K)                                         # 1, 4, 16 (of 64 slices) and 2 rounds
        assert f"kernel={KIND} " in d and "round_sync=0" in d and " ws=0 " in d, d
    d = _describe(16384, 28672, 8192, b_col=True, flags=ll.LL_FLAG_PRODUCER_CONSUMER)   # another kind
    assert f"kernel={KIND} " not in d and "round_sync=0" in d, d
    d = _describe(16384, 28672, 8192, b_col=True)                      # B K-contiguous, in place
    assert f"kernel={KIND} " in d and "packB=0" in d and "round_sync=1" in d, d
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "0")
    d = _describe(16384, 28672, 8192)
    assert "round_sync=0" in d and " ws=0 " in d, d
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "1")
    assert "round_sync=1" in _describe(8192, 8192, 1024)
    assert "round_sync=1" in _describe(4096, 8192, 8192)
    assert "round_sync=0" in _describe(4096, 4096, 4096)              # still needs two rounds


def _run_sync(A, B, C, sync, monkeypatch, bias=None, act=None):
    import torch
    import recsys_linear_layers_amd as ll
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "1" if sync else "0")
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    try:
        ll.gemm(A, B, out=C, bias=bias, act=act)
        torch.cuda.synchronize()
        ep = (ll.LL_EPI_BIAS if bias is not None else 0) | ll.ACTIVATIONS[act]
        d = ll.plan_for(A, B, C, 0, ep).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_ROUND_SYNC", raising=False)
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()
    assert f"kernel={KIND} " in d and f"round_sync={int(sync)}" in d, d
    return d


@pytest.mark.parametrize("act", [None, "gelu"])
def test_round_barrier_changes_no_bits(act, monkeypatch):
    """The round barrier only delays loads: with and without it the bits are
    the same.  8192 x 8704: 32 x 34 = 1088 tiles, four full rounds and a
    fifth of 64 tiles; checked against the oracle on 64-row strips and
    samples, plain and with bias + GELU."""
    import torch
    M, N, K = 8192, 8704, 256
    c = synth.gemm_case(M, N, K, seed=95 + (act is None), out_dtype="bf16", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    bias = None
    if act:
        bias = torch.from_numpy(np.random.default_rng(96).standard_normal(N).astype(np.float32)).cuda()
    C1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    C2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    d1 = _run_sync(A, B, C1, True, monkeypatch, bias, act)
    _run_sync(A, B, C2, False, monkeypatch, bias, act)
    assert torch.equal(C1, C2), d1
    got = to_f64(C1)
    rows, cols = sample_indices(M, N, 2048, 97, tile=(256, 256))
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    if act:
        ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act, cols=cols)
    acceptance.assert_close(got[rows, cols], ref, S, "bf16", f"samples {d1}", act=act)
    for r0, nr in strip_starts(M, 64, 98)[:3]:
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        if act:
            ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
        acceptance.assert_close(got[r0:r0 + nr], ref, S, "bf16", f"rows {r0}.. {d1}", act=act)


def _grouped(tin, tiles_m, tiles_n, group_m=8):
    """Tile (row, column) of grouped-order tile index tin, as the plan orders tiles."""
    per = group_m * tiles_n
    g, w = divmod(tin, per)
    first = g * group_m
    gsz = min(tiles_m - first, group_m)
    return first + w % gsz, w // gsz


def _tail_tiles(d, M, N):
    m = re.search(r"\btail=(\d+)x(\d+)", d)
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    nt = int(m.group(1))
    first = tiles_m * tiles_n - nt
    return [_grouped(first + i, tiles_m, tiles_n) for i in range(nt)], int(m.group(2))


def test_tail_split_selection():
    """A last round at most half full is split along K (up to 4 ways, at
    least 16 slices a split, splits x tiles within the grid); whole rounds,
    short K and other kinds are left alone."""
    import recsys_linear_layers_amd as ll
    assert " tail=128x2" in _describe(8191, 5003, 4099, b_col=True)   # 640 tiles: 2 rounds + 128
    assert " tail=65x3" in _describe(8448, 8448, 4096)                   # 1089 tiles: 4 rounds + 65
    for M, N, K in [(4096, 4096, 4096), (16384, 28672, 8192), (8192, 8192, 8192)]:
        assert " tail=0x1" in _describe(M, N, K)                         # whole rounds
    d = _describe(8448, 8448, 1984)                                      # 31 slices: splits would be short
    assert f"kernel={KIND} " in d and " tail=0x1" in d, d
    d = _describe(8191, 5003, 4099, b_col=True)
    assert int(d.split(" ws=")[1].split()[0]) >= 128 * 2 * 256 * 256 * 4, d


def _run_tail(A, B, C, monkeypatch, split, bias=None, act=None):
    import torch
    import recsys_linear_layers_amd as ll
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", KIND)
    if not split:
        monkeypatch.setenv("LL_GEMM_TAIL_SPLIT", "0")
    try:
        ll.gemm(A, B, out=C, bias=bias, act=act)
        torch.cuda.synchronize()
        ep = (ll.LL_EPI_BIAS if bias is not None else 0) | ll.ACTIVATIONS[act]
        d = ll.plan_for(A, B, C, 0, ep).describe()
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        monkeypatch.delenv("LL_GEMM_TAIL_SPLIT", raising=False)
        ll._plans.clear()
    assert f"kernel={KIND} " in d, d
    return d


@pytest.mark.parametrize("out,act", [("bf16", None), ("bf16", "gelu"), ("f32", None), ("f32", "silu")])
def test_tail_split_against_oracle(out, act, monkeypatch):
    """4300 x 4100 x 4096: 17 x 17 = 289 tiles, a last round of 33 split four
    ways (16 slices each), the ragged last tile row among them.  Every tail
    tile is checked on 64 sampled entries and a full row strip, every other
    tile on one entry; fp32 C with a row stride of N + 8."""
    import torch
    M, N, K = 4300, 4100, 4096
    c = synth.gemm_case(M, N, K, seed=311 + (act is not None) + 2 * (out == "f32"), out_dtype=out,
                        dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    bias = None
    if act:
        bias = torch.from_numpy(np.random.default_rng(312).standard_normal(N).astype(np.float32)).cuda()
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[out]
    big = torch.full((M, N + 8), float("nan"), dtype=dt, device="cuda")
    C = big[:, :N] if out == "f32" else torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    d = _run_tail(A, B, C, monkeypatch, True, bias, act)
    assert " tail=33x4" in d, d
    got = to_f64(C)
    tails, _ = _tail_tiles(d, M, N)
    rng = np.random.default_rng(313)
    rows, cols = per_tile_indices(M, N, (256, 256), 314)
    rows, cols = list(rows), list(cols)
    for tm, tn in tails:
        h, w = min(256, M - 256 * tm), min(256, N - 256 * tn)
        rows += list(256 * tm + rng.integers(0, h, 64))
        cols += list(256 * tn + rng.integers(0, w, 64))
    rows, cols = np.array(rows), np.array(cols)
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    if act:
        ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act, cols=cols)
    acceptance.assert_close(got[rows, cols], ref, S, out, f"tail samples {d}", act=act)
    for tm in sorted({tm for tm, _ in tails}):
        r0 = 256 * tm + 5 if 256 * tm + 5 < M else 256 * tm
        nr = min(4, M - r0)
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        if act:
            ref, S = oracle.epilogue(ref, S, bias.cpu().numpy(), act)
        acceptance.assert_close(got[r0:r0 + nr], ref, S, out, f"tail rows {r0}.. {d}", act=act)
    if out == "f32":
        assert torch.isnan(big[:, N:]).all()   # the padding columns are untouched


def test_tail_split_integer_inputs_bit_exact(monkeypatch):
    """With small integer inputs every partial sum is exact: the K-split tail
    tiles give the same bits as the unsplit kernel, and the oracle's."""
    import torch
    M, N, K = 4352, 4096, 2048
    c = synth.gemm_case(M, N, K, dist=("int", -4, 4), seed=315, out_dtype="f32")
    A, B = gemm_operands(c)
    C1 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    C2 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    d1 = _run_tail(A, B, C1, monkeypatch, True)
    d2 = _run_tail(A, B, C2, monkeypatch, False)
    assert " tail=16x2" in d1 and " tail=0x1" in d2, (d1, d2)
    assert torch.equal(C1, C2)
    tails, _ = _tail_tiles(d1, M, N)
    tm, tn = tails[-1]
    ref, _ = oracle.gemm_case(c, rows=(256 * tm, 8))
    assert np.array_equal(to_f64(C1)[256 * tm:256 * tm + 8], ref)


def test_b_prefetch_selection_and_bits(monkeypatch):
    """B is prefetched into L2 a slice ahead when its rows are 16384 elements
    or more apart and K >= 8192; the prefetch only warms the cache, so the
    bits are the same with and without it."""
    import torch
    import recsys_linear_layers_amd as ll
    assert "prefetch_b=1" in _describe(16384, 28672, 8192)              # FFN up
    for M, N, K in [(16384, 8192, 28672), (4096, 4096, 4096), (4096, 28672, 4096)]:
        assert "prefetch_b=0" in _describe(M, N, K), (M, N, K)          # FFN down, 4096^3, short K
    M, N, K = 2048, 16384, 1024
    c = synth.gemm_case(M, N, K, seed=321, out_dtype="bf16", dist=("normal", 0.0, 1.0))
    A, B = gemm_operands(c)
    outs, descs = [], []
    for on in ("1", "0"):
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        ll._plans.clear()
        monkeypatch.setenv("LL_GEMM_KIND", KIND)
        monkeypatch.setenv("LL_GEMM_PREFETCH_B", on)
        try:
            ll.gemm(A, B, out=C)
            torch.cuda.synchronize()
            descs.append(ll.plan_for(A, B, C).describe())
        finally:
            monkeypatch.delenv("LL_GEMM_KIND", raising=False)
            monkeypatch.delenv("LL_GEMM_PREFETCH_B", raising=False)
            ll._plans.clear()
        outs.append(C)
    assert "prefetch_b=1" in descs[0] and "prefetch_b=0" in descs[1], descs
    assert torch.equal(outs[0], outs[1])
    for r0, nr in strip_starts(M, 8, 322):
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        acceptance.assert_close(to_f64(outs[0][r0:r0 + nr]), ref, S, "bf16", f"rows {r0}.. {descs[0]}")
