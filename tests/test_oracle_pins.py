"""Pins of the fp64 oracle against things other than itself: exact rational
arithmetic on tiny inputs, numpy's float64 matmul, closed forms, integer
exactness, layout identities and the invariance of the user-once rewrite.
All CPU-only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import acceptance

U53 = 2.0 ** -53


def _mixed_bf16(rng, n):
    """bf16 patterns with random sign, exponent in [-12, 12] and mantissa."""
    m = rng.random(n, dtype=np.float32) + np.float32(1.0)
    e = rng.integers(-12, 13, n).astype(np.float32)
    s = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    return synth.f32_to_bf16_rne(s * m * np.exp2(e))


def _frac(bits):
    return [Fraction(float(v)) for v in synth.bf16_to_f32(bits)]


def _layout(rng, rows, cols, which):
    """Returns (buffer_size, row_stride, col_stride) for a rows x cols operand."""
    if which == "row":
        ld = cols + int(rng.integers(0, 3))
        return rows * ld, ld, 1
    ld = rows + int(rng.integers(0, 3))
    return cols * ld, 1, ld


def test_bruteforce_exact_rationals_all_shapes_1_to_8():
    rng = np.random.default_rng(1234)
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                la, lb = rng.choice(["row", "col"]), rng.choice(["row", "col"])
                na, sam, sak = _layout(rng, M, K, la)
                nb, sbk, sbn = _layout(rng, K, N, lb)
                A = _mixed_bf16(rng, na)
                B = _mixed_bf16(rng, nb)
                C, S = oracle.gemm(M, N, K, A, sam, sak, B, sbk, sbn)
                fa, fb = _frac(A), _frac(B)
                for i in range(M):
                    for j in range(N):
                        terms = [fa[i * sam + k * sak] * fb[k * sbk + j * sbn] for k in range(K)]
                        exact = sum(terms, Fraction(0))
                        sabs = sum((abs(t) for t in terms), Fraction(0))
                        tol = K * U53 * float(sabs) * 1.0001
                        assert abs(Fraction(C[i, j]) - exact) <= Fraction(tol), (M, N, K, i, j)
                        assert abs(Fraction(S[i, j]) - sabs) <= Fraction(tol), (M, N, K, i, j)


def test_matches_numpy_float64_matmul():
    rng = np.random.default_rng(7)
    for (M, N, K) in [(33, 17, 129), (64, 64, 64), (5, 300, 77)]:
        c = synth.gemm_case(M, N, K, seed=int(rng.integers(1 << 30)), dist=("normal", 0, 1.0))
        C, S = oracle.gemm_case(c)
        A = synth.bf16_to_f32(c.A).astype(np.float64).reshape(M, K)
        B = synth.bf16_to_f32(c.B).astype(np.float64).reshape(K, N)
        ref = A @ B
        Sref = np.abs(A) @ np.abs(B)
        assert np.all(np.abs(C - ref) <= 2 * K * U53 * Sref + 1e-300)
        assert np.allclose(S, Sref, rtol=4 * K * U53, atol=0)


def test_identity_and_permutation_exact():
    rng = np.random.default_rng(3)
    n = 40
    X = _mixed_bf16(rng, n * n)
    I = synth.f32_to_bf16_rne(np.eye(n, dtype=np.float32)).reshape(-1)
    Xf = synth.bf16_to_f32(X).astype(np.float64).reshape(n, n)
    C, _ = oracle.gemm(n, n, n, X, n, 1, I, n, 1)
    assert np.array_equal(C, Xf)
    C, _ = oracle.gemm(n, n, n, I, n, 1, X, n, 1)
    assert np.array_equal(C, Xf)
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    C, _ = oracle.gemm(n, n, n, synth.f32_to_bf16_rne(P).reshape(-1), n, 1, X, n, 1)
    assert np.array_equal(C, Xf[perm])
    # A.I with I column-major and A column-major
    C, _ = oracle.gemm(n, n, n, X, 1, n, I, 1, n)
    assert np.array_equal(C, Xf.T)


def test_rank1_closed_forms():
    rng = np.random.default_rng(5)
    M, N, K = 12, 9, 64
    u = _mixed_bf16(rng, M)
    v = _mixed_bf16(rng, N)
    one = synth.f32_to_bf16_rne(np.ones(1, dtype=np.float32))[0]
    A = np.repeat(u, K)                      # A[i][k] = u[i]
    B = np.tile(v, K)                        # B[k][j] = v[j]
    C, _ = oracle.gemm(M, N, K, A, K, 1, B, N, 1)
    uf = synth.bf16_to_f32(u).astype(np.float64)
    vf = synth.bf16_to_f32(v).astype(np.float64)
    assert np.array_equal(C, K * np.outer(uf, vf))
    # A = u a^T, B = b v^T  ->  C = (a.b) u v^T
    a = _mixed_bf16(rng, K)
    b = _mixed_bf16(rng, K)
    ua = synth.f32_to_bf16_rne((np.outer(uf, synth.bf16_to_f32(a))).astype(np.float32))
    # choose u = 1 so that u a^T stays exactly representable
    A = np.tile(a, M)                        # A[i][k] = a[k]
    B = np.repeat(b, N)                      # B[k][j] = b[k]
    C, S = oracle.gemm(M, N, K, A, K, 1, B, N, 1)
    fa, fb = _frac(a), _frac(b)
    dot = sum((x * y for x, y in zip(fa, fb)), Fraction(0))
    sabs = sum((abs(x * y) for x, y in zip(fa, fb)), Fraction(0))
    assert np.all(np.abs(C - float(dot)) <= K * U53 * float(sabs))
    assert one == 0x3F80 and ua.size == M * K


def test_integer_valued_inputs_are_exact():
    for (M, N, K) in [(16, 16, 16), (31, 45, 257), (8, 8, 4096)]:
        c = synth.gemm_case(M, N, K, dist=("int", -4, 4), seed=M * N + K)
        C, _ = oracle.gemm_case(c)
        A = synth.bf16_to_f32(c.A).astype(np.int64).reshape(M, K)
        B = synth.bf16_to_f32(c.B).astype(np.int64).reshape(K, N)
        assert np.array_equal(C, (A @ B).astype(np.float64))


def test_column_major_b_equals_row_major_copy():
    M, N, K = 23, 31, 70
    c = synth.gemm_case(M, N, K, seed=9, b_col_major=True, lda=K + 3, ldb=K + 5)
    C1, S1 = oracle.gemm_case(c)
    Bt = c.B.reshape(N, K + 5)[:, :K]          # [N][K]
    Brow = np.ascontiguousarray(Bt.T).reshape(-1)  # [K][N]
    C2, S2 = oracle.gemm(M, N, K, c.A, K + 3, 1, Brow, N, 1)
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def test_entries_and_row_strips_agree_with_full():
    c = synth.gemm_case(50, 60, 300, seed=4, dist=("normal", 0, 1.0))
    C, S = oracle.gemm_case(c)
    Cs, Ss = oracle.gemm_case(c, rows=(17, 9))
    assert np.array_equal(Cs, C[17:26]) and np.array_equal(Ss, S[17:26])
    rng = np.random.default_rng(0)
    r = rng.integers(0, 50, 200)
    col = rng.integers(0, 60, 200)
    e, es = oracle.gemm_case_entries(c, r, col)
    assert np.array_equal(e, C[r, col]) and np.array_equal(es, S[r, col])


def _lc_dense(R, C, Nu, Ni, D, Mo, rng, dist):
    if dist == "int":
        mk = lambda n: synth.f32_to_bf16_rne(rng.integers(-3, 4, n).astype(np.float32))
    else:
        mk = lambda n: _mixed_bf16(rng, n)
    return mk(R * Nu * D), mk(R * C * Ni * D), mk((Nu + Ni) * Mo)


def _lc_strides(R, C, Nu, Ni, D, Mo):
    return dict(su_r=Nu * D, su_n=D, si_r=C * Ni * D, si_c=Ni * D, si_n=D, sw_n=Mo)


def test_lincomp_naive_matches_numpy_on_stacked_input():
    rng = np.random.default_rng(11)
    R, C, Nu, Ni, D, Mo = 3, 4, 5, 7, 6, 3
    user, item, W = _lc_dense(R, C, Nu, Ni, D, Mo, rng, "mixed")
    st = _lc_strides(R, C, Nu, Ni, D, Mo)
    pairs = [(r, c) for r in range(R) for c in range(C)]
    Y, S = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), user, item, W, st, pairs)
    u = synth.bf16_to_f32(user).astype(np.float64).reshape(R, Nu, D)
    it = synth.bf16_to_f32(item).astype(np.float64).reshape(R, C, Ni, D)
    w = synth.bf16_to_f32(W).astype(np.float64).reshape(Nu + Ni, Mo)
    for p, (r, c) in enumerate(pairs):
        X = np.concatenate([u[r], it[r, c]], axis=0)
        ref = w.T @ X
        Sref = np.abs(w.T) @ np.abs(X)
        assert np.all(np.abs(Y[p] - ref) <= 2 * (Nu + Ni) * U53 * Sref)
        assert np.allclose(S[p], Sref, rtol=4 * (Nu + Ni) * U53, atol=0)
    # exact rationals for one candidate
    fu, fi, fw = _frac(user), _frac(item), _frac(W)
    r, c = 2, 1
    for m in range(Mo):
        for d in range(D):
            terms = [fw[n * Mo + m] * fu[r * Nu * D + n * D + d] for n in range(Nu)]
            terms += [fw[(Nu + n) * Mo + m] * fi[r * C * Ni * D + c * Ni * D + n * D + d]
                      for n in range(Ni)]
            ex = sum(terms, Fraction(0))
            sa = sum((abs(t) for t in terms), Fraction(0))
            p = pairs.index((r, c))
            assert abs(Fraction(Y[p, m, d]) - ex) <= Fraction((Nu + Ni) * U53 * float(sa))


def test_lincomp_dedup_invariance():
    rng = np.random.default_rng(12)
    R, C, Nu, Ni, D, Mo = 2, 3, 16, 24, 8, 5
    st = _lc_strides(R, C, Nu, Ni, D, Mo)
    pairs = [(r, c) for r in range(R) for c in range(C)]
    user, item, W = _lc_dense(R, C, Nu, Ni, D, Mo, rng, "mixed")
    Yn, S = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), user, item, W, st, pairs)
    Yd = oracle.lincomp_dedup((R, C, Nu, Ni, D, Mo), user, item, W, st, pairs)
    assert np.all(np.abs(Yn - Yd) <= 2 * (Nu + Ni) * U53 * S)
    user, item, W = _lc_dense(R, C, Nu, Ni, D, Mo, rng, "int")
    Yn = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), user, item, W, st, pairs, bound=False)
    Yd = oracle.lincomp_dedup((R, C, Nu, Ni, D, Mo), user, item, W, st, pairs)
    assert np.array_equal(Yn, Yd)


def test_lincomp_selector_special_cases():
    rng = np.random.default_rng(13)
    R, C, Nu, Ni, D, Mo = 2, 3, 6, 4, 5, 4
    st = _lc_strides(R, C, Nu, Ni, D, Mo)
    pairs = [(r, c) for r in range(R) for c in range(C)]
    user, item, _ = _lc_dense(R, C, Nu, Ni, D, Mo, rng, "mixed")
    uf = synth.bf16_to_f32(user).astype(np.float64).reshape(R, Nu, D)
    itf = synth.bf16_to_f32(item).astype(np.float64).reshape(R, C, Ni, D)
    # W = [E; 0] with E selecting user rows sel_u[m]
    sel_u = [5, 0, 3, 3]
    Wf = np.zeros((Nu + Ni, Mo), dtype=np.float32)
    for m, n in enumerate(sel_u):
        Wf[n, m] = 1.0
    Y = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), user, item, synth.f32_to_bf16_rne(Wf), st,
                             pairs, bound=False)
    for p, (r, c) in enumerate(pairs):
        assert np.array_equal(Y[p], uf[r][sel_u])
    # W = [0; E] selecting item rows
    sel_i = [1, 3, 0, 2]
    Wf[:] = 0
    for m, n in enumerate(sel_i):
        Wf[Nu + n, m] = 1.0
    Y = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), user, item, synth.f32_to_bf16_rne(Wf), st,
                             pairs, bound=False)
    for p, (r, c) in enumerate(pairs):
        assert np.array_equal(Y[p], itf[r, c][sel_i])
    # zero user block: the user rows contribute exactly nothing
    _, _, W = _lc_dense(R, C, Nu, Ni, D, Mo, rng, "mixed")
    zu = np.zeros_like(user)
    Y = oracle.lincomp_naive((R, C, Nu, Ni, D, Mo), zu, item, W, st, pairs, bound=False)
    Wi = W.reshape(Nu + Ni, Mo)[Nu:].reshape(-1)
    for p, (r, c) in enumerate(pairs):
        it = item.reshape(R, C, Ni * D)[r, c]
        ref, _ = oracle.gemm(Mo, D, Ni, Wi, 1, Mo, it, D, 1)   # A = Wi^T (column-major view)
        assert np.array_equal(Y[p], ref)


def test_acceptance_rne_passes_truncation_fails():
    # values needing rounding to 8 significant bits; K = 1 so S = |ref|
    x = np.array([1 + 2 ** -7 - 2 ** -20, -(3 + 0.9 * 2 ** -6), 1000.9, 2 ** -10 * 1.99],
                 dtype=np.float32)
    ref = x.astype(np.float64)
    S = np.abs(ref)
    rne = synth.bf16_to_f32(synth.f32_to_bf16_rne(x)).astype(np.float64)
    trunc = synth.bf16_to_f32((x.view(np.uint32) >> 16).astype(np.uint16)).astype(np.float64)
    assert acceptance.check(rne, ref, S, "bf16")[0]
    assert not acceptance.check(trunc, ref, S, "bf16")[0]
    # fp32 bound
    z = np.zeros_like(ref)
    assert acceptance.check(z + 0.9e-6, z, z, "f32")[0]
    assert not acceptance.check(z + 2e-6, z, z, "f32")[0]
    assert acceptance.check(ref + 0.9e-3 * S, ref, S, "f32")[0]
    assert not acceptance.check(ref + 1.1e-3 * S + 1e-6, ref, S, "f32")[0]
    bad = ref.copy()
    bad[1] = np.nan
    assert not acceptance.check(bad, ref, S, "f32")[0]


def test_synth_rne_and_determinism():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7 - 2 ** -20, -2.0, 0.0],
                 dtype=np.float32)
    assert list(synth.f32_to_bf16_rne(x)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0]
    a = synth.bf16_tensor(3 * synth.CHUNK + 17, "normal", 0, 1.0, seed=42, tensor=3)
    b = synth.bf16_tensor(3 * synth.CHUNK + 17, "normal", 0, 1.0, seed=42, tensor=3)
    assert np.array_equal(a, b)
    c = synth.bf16_tensor(synth.CHUNK + 5, "normal", 0, 1.0, seed=42, tensor=3)
    assert np.array_equal(c, a[: synth.CHUNK + 5])
    d = synth.bf16_tensor(100, "int", -4, 4, seed=1)
    f = synth.bf16_to_f32(d)
    assert f.min() >= -4 and f.max() <= 4 and np.all(f == np.round(f))


def test_golden_fixture():
    """tests/golden/gemm_int_7x5x9.txt: written by tests/golden/make_golden.py from
    the oracle; integer inputs, so the closed form (int64 matmul) must agree too."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "gemm_int_7x5x9.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    M, N, K = (int(v) for v in rows[0])
    A = np.array([int(v) for v in rows[1]], dtype=np.int64).reshape(M, K)
    B = np.array([int(v) for v in rows[2]], dtype=np.int64).reshape(K, N)
    C = np.array([float(v) for v in rows[3]]).reshape(M, N)
    assert np.array_equal(A @ B, C.astype(np.int64))
    Ab = synth.f32_to_bf16_rne(A.astype(np.float32)).reshape(-1)
    Bb = synth.f32_to_bf16_rne(B.astype(np.float32)).reshape(-1)
    Co, _ = oracle.gemm(M, N, K, Ab, K, 1, Bb, N, 1)
    assert np.array_equal(Co, C)


# ---------------------------------------------------------------------------
# fp16 operands
# ---------------------------------------------------------------------------

def test_f16_widening_matches_numpy_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("bits,value", [(0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
                                        (0x0400, 2.0 ** -14), (0x03FF, 1023 * 2.0 ** -24), (0x3555, 1365 / 4096),
                                        (0x8000, -0.0), (0x7C00, float("inf"))])
def test_f16_widening_closed_forms(bits, value):
    got = oracle.widen(np.array([bits], dtype=np.uint16), "f16")[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def _mixed_f16(rng, n):
    """fp16 patterns with random sign, exponent in [-20, 12] (subnormals included) and mantissa."""
    m = rng.random(n, dtype=np.float32) + np.float32(1.0)
    e = rng.integers(-20, 13, n).astype(np.float32)
    s = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    return synth.f32_to_f16_rne(s * m * np.exp2(e))


def test_f16_bruteforce_exact_rationals():
    rng = np.random.default_rng(4321)
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 9):
                la, lb = rng.choice(["row", "col"]), rng.choice(["row", "col"])
                na, sam, sak = _layout(rng, M, K, la)
                nb, sbk, sbn = _layout(rng, K, N, lb)
                A = _mixed_f16(rng, na)
                B = _mixed_f16(rng, nb)
                C, S = oracle.gemm(M, N, K, A, sam, sak, B, sbk, sbn, fmt="f16")
                fa = [Fraction(float(v)) for v in A.view(np.float16)]
                fb = [Fraction(float(v)) for v in B.view(np.float16)]
                for i in range(M):
                    for j in range(N):
                        terms = [fa[i * sam + k * sak] * fb[k * sbk + j * sbn] for k in range(K)]
                        exact = sum(terms, Fraction(0))
                        sabs = sum((abs(t) for t in terms), Fraction(0))
                        tol = K * U53 * float(sabs) * 1.0001
                        assert abs(Fraction(C[i, j]) - exact) <= Fraction(tol), (M, N, K, i, j)
                        assert abs(Fraction(S[i, j]) - sabs) <= Fraction(tol), (M, N, K, i, j)


def test_f16_entries_agree_with_rows():
    c = synth.gemm_case(37, 29, 70, seed=5, in_dtype="f16", dist=("normal", 0, 1.0))
    C, S = oracle.gemm_case(c)
    rows = np.array([0, 36, 5, 17], dtype=np.int64)
    cols = np.array([0, 28, 3, 11], dtype=np.int64)
    e, Se = oracle.gemm_case_entries(c, rows, cols)
    assert np.array_equal(e, C[rows, cols]) and np.array_equal(Se, S[rows, cols])


def test_f16_case_is_not_read_as_bf16():
    # the same bits decoded as bf16 give other values: the format reaches the oracle
    c = synth.gemm_case(8, 8, 8, seed=6, in_dtype="f16", dist=("normal", 0, 1.0))
    C16, _ = oracle.gemm_case(c)
    Cb, _ = oracle.gemm(8, 8, 8, c.A, c.sam, c.sak, c.B, c.sbk, c.sbn, fmt="bf16")
    A = c.A.view(np.float16).astype(np.float64).reshape(8, 8)
    B = c.B.view(np.float16).astype(np.float64).reshape(8, 8)
    assert np.allclose(C16, A @ B, rtol=1e-12, atol=1e-12)
    assert not np.allclose(Cb, C16)


def test_f16_acceptance_passes_rne_fails_truncation():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal(4096) * 100.0
    S = np.zeros_like(ref)
    rne = ref.astype(np.float32).astype(np.float16).astype(np.float64)
    assert acceptance.check(rne, ref, S, "f16")[0]
    # truncation toward zero: clear the bits below fp16's last place
    r32 = ref.astype(np.float32)
    f16 = r32.astype(np.float16)
    up = np.abs(f16.astype(np.float32)) > np.abs(r32)
    trunc = np.where(up, np.nextafter(f16, np.float16(0)), f16).astype(np.float64)
    assert not acceptance.check(trunc, ref, S, "f16")[0]


# ---------------------------------------------------------------------------
# GEMM epilogue: bias and activation
# ---------------------------------------------------------------------------

def test_epilogue_activations_match_scipy():
    from scipy.special import expit, ndtr
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(2000) * 3.0, np.linspace(-40, 40, 801), [0.0, -0.0, 1e-300]])
    C = x.reshape(1, -1)
    for act, ref in [("relu", np.maximum(x, 0.0)), ("gelu", x * ndtr(x)), ("silu", x * expit(x)), (None, x)]:
        got, _ = oracle.epilogue(C, None, None, act)
        np.testing.assert_allclose(got[0], ref, rtol=1e-12, atol=1e-300)  # two fp64 libraries for Phi


def test_epilogue_bias_is_added_exactly_and_counted_in_S():
    rng = np.random.default_rng(22)
    C = rng.standard_normal((3, 7))
    S = np.abs(C) * 2
    bias = rng.standard_normal(7).astype(np.float32)
    got, S2 = oracle.epilogue(C, S, bias, None)
    assert np.array_equal(got, C + bias.astype(np.float64))
    assert np.array_equal(S2, S + np.abs(bias.astype(np.float64)))
    # sampled entries take their column's bias
    cols = np.array([6, 0, 3])
    g1, _ = oracle.epilogue(C[0, cols], S[0, cols], bias, "gelu", cols=cols)
    g2, _ = oracle.epilogue(C, S, bias, "gelu")
    assert np.array_equal(g1, g2[0, cols])


def test_epilogue_closed_forms():
    C = np.array([[0.0, 1.0, -1.0, 50.0, -50.0]])
    g, _ = oracle.epilogue(C, None, None, "gelu")
    assert g[0, 0] == 0.0 and g[0, 3] == 50.0 and abs(g[0, 4]) < 1e-300 * 1e300 * 1e-500 + 1e-200
    assert abs(g[0, 1] - 0.8413447460685429) < 1e-15 and abs(g[0, 2] + 0.15865525393145707) < 1e-15
    s, _ = oracle.epilogue(C, None, None, "silu")
    assert s[0, 0] == 0.0 and abs(s[0, 1] - 1 / (1 + np.exp(-1.0))) < 1e-16 and s[0, 3] == 50.0


def test_activation_bound_is_what_the_slope_allows():
    # a sum off by e moves GELU by at most 1.13 e: a shifted sum at the bound passes, 3x the bound fails
    rng = np.random.default_rng(23)
    z = rng.standard_normal(5000) * 2
    S = np.abs(z) * 10 + 1
    e = 1e-3 * S + 1e-6
    ref, _ = oracle.epilogue(z.reshape(1, -1), None, None, "gelu")
    near, _ = oracle.epilogue((z + e).reshape(1, -1), None, None, "gelu")
    far, _ = oracle.epilogue((z + 3 * e).reshape(1, -1), None, None, "gelu")
    assert acceptance.check(near[0], ref[0], S, "f32", "gelu")[0]
    assert not acceptance.check(far[0], ref[0], S, "f32", "gelu")[0]


def test_lincomp_epilogue_bias_runs_along_compressed_rows():
    """W = [E; 0] selects user rows exactly (integer inputs), so
    act(Y + bias) has a closed form per (m, d): relu(user[r][sel(m)][d] + b[m]).
    A bias applied along d instead of m, or not at all, fails it."""
    R, C, Nu, Ni, D, Mo = 2, 3, 8, 4, 24, 8
    c = synth.lincomp_case(R, C, Nu, Ni, D, Mo, x_dist=("int", -3, 3), seed=91, name="epi_sel")
    sel = np.array([5, 0, 7, 2, 2, 6, 1, 3])
    W = np.zeros((Nu + Ni, Mo), dtype=np.float32)
    W[sel, np.arange(Mo)] = 1.0
    c.W = synth.f32_to_bf16_rne(W.reshape(-1))
    bias = (np.arange(Mo, dtype=np.float32) - 3.5) * 2.0
    pairs = [(r, k) for r in range(R) for k in range(C)]
    Y, S = oracle.lincomp_case(c, pairs)
    got, Sb = oracle.lincomp_epilogue(Y, S, bias, "relu")
    user = synth.bf16_to_f32(c.user).astype(np.float64).reshape(R, Nu, D)
    want = np.stack([np.maximum(user[r][sel] + bias[:, None], 0.0) for r, _ in pairs])
    assert np.array_equal(got, want)
    assert np.array_equal(Sb, S + np.abs(bias)[None, :, None])
    wrong = np.stack([np.maximum(user[r][sel] + np.resize(bias, D)[None, :], 0.0) for r, _ in pairs])
    assert not np.array_equal(got, wrong)
    none, _ = oracle.lincomp_epilogue(Y, S, None, "relu")
    assert not np.array_equal(got, none)
    # no activation and no bias is the identity
    ident, Si = oracle.lincomp_epilogue(Y, S, None, None)
    assert np.array_equal(ident, Y) and np.array_equal(Si, S)
