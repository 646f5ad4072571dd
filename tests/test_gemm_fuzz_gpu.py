"""Seeded random GEMM cases on the GPU against the fp64 oracle, element by
element: sizes, operand layouts and leading dimensions, input and output
types, epilogue and plan flags all drawn at random, so that combinations the
parametrised tests do not list are covered too.  Every draw is reproducible
from the case index."""
import numpy as np
import pytest

import oracle
import synth
from helpers import to_f64
from oracle import acceptance
from synth.device import gemm_operands as gemm_operands_t, to_device

pytestmark = pytest.mark.gpu

N_CASES = 160


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    small = rng.random() < 0.3
    M = int(rng.integers(1, 40 if small else 521))
    N = int(rng.integers(1, 40 if small else 521))
    K = int(rng.integers(1, 40 if small else 801))
    in_dtype = str(rng.choice(["bf16", "f16"]))
    out = str(rng.choice(["f32", in_dtype]))
    a_col, b_col = bool(rng.random() < 0.4), bool(rng.random() < 0.4)
    pad_a, pad_b = int(rng.choice([0, 0, 1, 3, 8])), int(rng.choice([0, 0, 2, 5, 8]))
    act = rng.choice([None, None, "relu", "gelu", "silu"])
    bias = bool(rng.random() < 0.5) or act is not None and rng.random() < 0.5
    flags = int(rng.choice([0, 0, 0, 0x1, 0x2, 0x3, 0x4, 0x8]))
    return dict(M=M, N=N, K=K, in_dtype=in_dtype, out=out, a_col=a_col, b_col=b_col, pad_a=pad_a,
                pad_b=pad_b, act=act, bias=bias, flags=flags, seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    _check(i, _draw(i))


N_SQUARE = 40


@pytest.mark.parametrize("i", range(N_SQUARE))
def test_random_case_square_kind(i, monkeypatch):
    """The 256x256 kind with one loading wave per SIMD, forced on random
    cases (no fused epilogue: that kind has none, and the plan would fall back
    to another)."""
    import recsys_linear_layers_amd as ll
    d = _draw(N_CASES + i)
    d["act"], d["bias"] = None, False
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ8_LW4")
    try:
        _check(N_CASES + i, d, want_kind="KIND_SQ8_LW4")
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()


N_SQ4 = 40


@pytest.mark.parametrize("i", range(N_SQ4))
def test_random_case_hand_ordered_kind(i, monkeypatch):
    """The hand-ordered 256x256 kind forced on random cases it applies to: A
    row-major (any leading dimension: a misaligned one is packed K-contiguous),
    B row-major (same, packed N-contiguous), K a multiple of 64; bias and
    activation as drawn."""
    import recsys_linear_layers_amd as ll
    d = _draw(N_CASES + N_SQUARE + i)
    rng = np.random.default_rng(5000 + i)
    d["K"] = 64 * int(rng.integers(1, 13))
    d["a_col"], d["b_col"] = False, False
    d["flags"] = 0
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    try:
        _check(N_CASES + N_SQUARE + i, d, want_kind="KIND_SQ4_HO")
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()


N_SQ4_BK = 16


@pytest.mark.parametrize("i", range(N_SQ4_BK))
def test_random_case_hand_ordered_b_k_contiguous(i, monkeypatch):
    """The hand-ordered kind's variant for a K-contiguous B (C = X W^T) forced
    on random cases: B column-major with any leading dimension (a misaligned
    one is packed, still K-contiguous), K a multiple of 64 for even i; for odd
    i any K with both operands packed (their zero columns past K meet in the
    last 64-deep slice); bias, activation and output type as drawn."""
    import recsys_linear_layers_amd as ll
    d = _draw(N_CASES + N_SQUARE + N_SQ4 + 1000 + i)
    rng = np.random.default_rng(8000 + i)
    d["M"] = int(rng.integers(1, 1100))
    d["N"] = int(rng.integers(1, 1100))
    d["a_col"], d["b_col"] = False, True
    if i % 2 == 0:
        d["K"] = 64 * int(rng.integers(1, 13))
        d["flags"] = 0
    else:
        d["K"] = 64 * int(rng.integers(0, 9)) + int(rng.integers(1, 64))
        d["flags"] = ll.LL_FLAG_PACK_A | ll.LL_FLAG_PACK_B
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    try:
        _check(N_CASES + N_SQUARE + N_SQ4 + 1000 + i, d, want_kind="KIND_SQ4_HO", want="B:K-major")
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()


N_SQ4_AM = 16


@pytest.mark.parametrize("i", range(N_SQ4_AM))
def test_random_case_hand_ordered_a_m_contiguous(i, monkeypatch):
    """The hand-ordered kind's variants for an M-contiguous A (C = X^T Y)
    forced on random cases: M a multiple of 8 (A read in place), B either way
    as drawn, any K (a K-contiguous B is then packed when K is not a multiple
    of 64); bias, activation and output type as drawn."""
    import recsys_linear_layers_amd as ll
    d = _draw(N_CASES + N_SQUARE + N_SQ4 + 2000 + i)
    rng = np.random.default_rng(8500 + i)
    d["M"] = 8 * int(rng.integers(1, 138))
    d["N"] = int(rng.integers(1, 1100))
    d["K"] = int(rng.integers(1, 700))
    d["a_col"] = True
    d["pad_a"] = 8 * int(rng.integers(0, 3))
    d["flags"] = ll.LL_FLAG_PACK_B if (d["b_col"] and d["K"] % 64) else 0
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    try:
        _check(N_CASES + N_SQUARE + N_SQ4 + 2000 + i, d, want_kind="KIND_SQ4_HO", want="A:M-major")
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()


N_SQ4_TAIL = 30


@pytest.mark.parametrize("i", range(N_SQ4_TAIL))
def test_random_case_hand_ordered_k_tail(i, monkeypatch):
    """The hand-ordered kind forced on random cases whose K is not a multiple
    of 64, with A packed (it reads whole 64-deep slices, which is exact only
    against a packed A's zero columns).  Sizes reach past four tiles so that
    interior tiles take the staged epilogue when N allows 16-byte rows; bias
    and activation as drawn."""
    import recsys_linear_layers_amd as ll
    d = _draw(N_CASES + N_SQUARE + N_SQ4 + i)
    rng = np.random.default_rng(7000 + i)
    d["M"] = int(rng.integers(1, 1100))
    d["N"] = 8 * int(rng.integers(1, 138)) if rng.random() < 0.6 else int(rng.integers(1, 1100))
    d["K"] = 64 * int(rng.integers(0, 9)) + int(rng.integers(1, 64))
    d["a_col"], d["b_col"] = False, False
    d["flags"] = ll.LL_FLAG_PACK_A
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    try:
        _check(N_CASES + N_SQUARE + N_SQ4 + i, d, want_kind="KIND_SQ4_HO")
    finally:
        monkeypatch.delenv("LL_GEMM_KIND", raising=False)
        ll._plans.clear()


N_FEATURES = 8


@pytest.mark.parametrize("i", range(N_FEATURES))
def test_random_case_hand_ordered_features(i, monkeypatch):
    """The hand-ordered kind on random shapes of more than one round of
    256x256 tiles, with its round barrier, its K-split last round and its B
    prefetch each forced on or off at random (bias and activation and the
    output type drawn too); sampled against the oracle: one entry in every
    tile, 32 in each tile of the last round, and row strips."""
    import torch
    import recsys_linear_layers_amd as ll
    from helpers import per_tile_indices, strip_starts
    rng = np.random.default_rng(9000 + i)
    sync, tail, pf = str(i & 1), str((i >> 1) & 1), str((i >> 2) & 1)   # every combination once
    while True:   # with the tail split on, a last round small enough to split
        M, N = int(rng.integers(4100, 6200)), int(rng.integers(4100, 6200))
        if tail == "0" or 0 < (-(-M // 256) * -(-N // 256)) % 256 <= 128:
            break
    K = 64 * int(rng.integers(32, 65))
    out = str(rng.choice(["bf16", "f32"]))
    act = rng.choice([None, "relu", "gelu", "silu"])
    use_bias = bool(rng.random() < 0.6)
    c = synth.gemm_case(M, N, K, seed=9100 + i, out_dtype=out, dist=("normal", 0.0, 1.0))
    A, B = gemm_operands_t(c)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    bias = (torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda() if use_bias else None)
    ll._plans.clear()
    for k, v in (("LL_GEMM_KIND", "KIND_SQ4_HO"), ("LL_GEMM_ROUND_SYNC", sync), ("LL_GEMM_TAIL_SPLIT", tail),
                 ("LL_GEMM_PREFETCH_B", pf)):
        monkeypatch.setenv(k, v)
    try:
        ll.gemm(A, B, out=C, bias=bias, act=act)
        torch.cuda.synchronize()
        ep = (ll.LL_EPI_BIAS if bias is not None else 0) | ll.ACTIVATIONS[act]
        d = ll.plan_for(A, B, C, 0, ep).describe()
    finally:
        for k in ("LL_GEMM_KIND", "LL_GEMM_ROUND_SYNC", "LL_GEMM_TAIL_SPLIT", "LL_GEMM_PREFETCH_B"):
            monkeypatch.delenv(k, raising=False)
        ll._plans.clear()
    what = f"features case {i}: {M}x{N}x{K} {out} act={act} bias={use_bias} {d}"
    assert "kernel=KIND_SQ4_HO " in what and f"round_sync={sync}" in d and f"prefetch_b={pf}" in d, what
    assert ("tail=0x1" in d) == (tail == "0"), what
    got = to_f64(C)
    rows, cols = per_tile_indices(M, N, (256, 256), 9200 + i)
    tiles_m, tiles_n = -(-M // 256), -(-N // 256)
    last = (tiles_m * tiles_n) % 256
    extra_r, extra_c = [], []
    for t in range(tiles_m * tiles_n - last, tiles_m * tiles_n):
        per, (gid, w) = 8 * tiles_n, divmod(t, 8 * tiles_n)
        gsz = min(tiles_m - 8 * gid, 8)
        tm, tn = 8 * gid + w % gsz, w // gsz
        h, wd = min(256, M - 256 * tm), min(256, N - 256 * tn)
        extra_r += list(256 * tm + rng.integers(0, h, 32))
        extra_c += list(256 * tn + rng.integers(0, wd, 32))
    rows, cols = np.concatenate([rows, extra_r]).astype(np.int64), np.concatenate([cols, extra_c]).astype(np.int64)
    ref, S = oracle.gemm_case_entries(c, rows, cols)
    if bias is not None or act is not None:
        ref, S = oracle.epilogue(ref, S, None if bias is None else bias.cpu().numpy(), act, cols=cols)
    acceptance.assert_close(got[rows, cols], ref, S, out, what, act=act)
    for r0, nr in strip_starts(M, 4, 9300 + i):
        ref, S = oracle.gemm_case(c, rows=(r0, nr))
        if bias is not None or act is not None:
            ref, S = oracle.epilogue(ref, S, None if bias is None else bias.cpu().numpy(), act)
        acceptance.assert_close(got[r0:r0 + nr], ref, S, out, f"{what} rows {r0}..", act=act)


def _check(i, d, want_kind=None, want=None):
    import torch
    import recsys_linear_layers_amd as ll
    M, N, K = d["M"], d["N"], d["K"]
    what = f"case {i}: {d}"
    # A: row-major [M][lda] or column-major [K][lda]; B: row-major [K][ldb] or column-major [N][ldb]
    if d["a_col"]:
        lda = M + d["pad_a"]
        A_bits = synth.bf16_tensor(K * lda, "uniform", -1.0, 1.0, seed=d["seed"], tensor=0, fmt=d["in_dtype"])
        sam, sak = 1, lda
    else:
        lda = K + d["pad_a"]
        A_bits = synth.bf16_tensor(M * lda, "uniform", -1.0, 1.0, seed=d["seed"], tensor=0, fmt=d["in_dtype"])
        sam, sak = lda, 1
    if d["b_col"]:
        ldb = K + d["pad_b"]
        B_bits = synth.bf16_tensor(N * ldb, "uniform", -1.0, 1.0, seed=d["seed"], tensor=1, fmt=d["in_dtype"])
        sbk, sbn = 1, ldb
    else:
        ldb = N + d["pad_b"]
        B_bits = synth.bf16_tensor(K * ldb, "uniform", -1.0, 1.0, seed=d["seed"], tensor=1, fmt=d["in_dtype"])
        sbk, sbn = ldb, 1
    A = to_device(A_bits, (M, K), (sam, sak), "cuda", d["in_dtype"])
    B = to_device(B_bits, (K, N), (sbk, sbn), "cuda", d["in_dtype"])
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[d["out"]]
    C = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    bias = None
    if d["bias"]:
        bias = torch.from_numpy(np.random.default_rng(d["seed"]).standard_normal(N).astype(np.float32)).cuda()
    if d["flags"] & ll.LL_FLAG_COOPERATIVE and (bias is not None or d["act"] is not None):
        with pytest.raises(ll.LLError) as e:
            ll.gemm(A, B, out=C, flags=d["flags"], bias=bias, act=d["act"])
        assert e.value.status == ll.LL_ERR_UNSUPPORTED, what
        return
    ll.gemm(A, B, out=C, flags=d["flags"], bias=bias, act=d["act"])
    torch.cuda.synchronize()
    if want_kind is not None or want is not None:
        desc = ll.plan_for(A, B, C, d["flags"]).describe()
        assert want_kind is None or f"kernel={want_kind} " in desc, what
        assert want is None or want in desc, (what, desc)
    ref, S = oracle.gemm(M, N, K, A_bits, sam, sak, B_bits, sbk, sbn, fmt=d["in_dtype"])
    if bias is not None or d["act"] is not None:
        ref, S = oracle.epilogue(ref, S, None if bias is None else bias.cpu().numpy(), d["act"])
    acceptance.assert_close(to_f64(C), ref, S, d["out"], what, act=d["act"])
