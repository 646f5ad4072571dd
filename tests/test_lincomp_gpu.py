"""Linear-compression parity on the GPU against the per-candidate fp64 oracle
(which stacks the request's user rows above each candidate's item rows)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import lincomp_operands, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _run(case, y_dtype="bf16", flags=0):
    import torch
    import recsys_linear_layers_amd as ll
    R, C, D, Mo = case.R, case.C, case.D, case.Mo
    user, item, W = lincomp_operands(case)
    dt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    Y = torch.full((R, C, Mo, D), float("nan"), dtype=dt, device="cuda")
    ll.lincomp(user, item, W, out=Y, flags=flags)
    torch.cuda.synchronize()
    return to_f64(Y)


def _run_stacked(case, y_dtype="bf16"):
    """The layer's original input: every candidate's [user rows; item rows]
    materialised in one tensor X [R][C][Nu+Ni][D]."""
    import torch
    import recsys_linear_layers_amd as ll
    R, C, D, Mo, Nu = case.R, case.C, case.D, case.Mo, case.Nu
    user, item, W = lincomp_operands(case)
    X = torch.cat([user[:, None].expand(R, C, Nu, D), item], dim=2).contiguous()
    del item
    dt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    Y = torch.full((R, C, Mo, D), float("nan"), dtype=dt, device="cuda")
    ll.lincomp_stacked(X, W, Nu, out=Y)
    torch.cuda.synchronize()
    return to_f64(Y)


def _check(case, pairs=None, y_dtype="bf16", flags=0, stacked=False):
    Y = _run_stacked(case, y_dtype) if stacked else _run(case, y_dtype, flags)
    pairs = pairs or [(r, c) for r in range(case.R) for c in range(case.C)]
    ref, S = oracle.lincomp_case(case, pairs)
    got = np.stack([Y[r, c] for r, c in pairs])
    acceptance.assert_close(got, ref, S, y_dtype, case.name)
    return Y


def test_small_workload_full():
    _check(synth.lincomp_workload("lincomp_small"))


@pytest.mark.parametrize("Nu,Ni,D,Mo", [(40, 24, 72, 24), (256, 64, 128, 64), (8, 200, 8, 8),
                                        (64, 64, 264, 72)])
def test_ragged_dims(Nu, Ni, D, Mo):
    c = synth.lincomp_case(2, 3, Nu, Ni, D, Mo, seed=40 + Nu + Ni, name=f"lc{Nu}_{Ni}_{D}_{Mo}")
    _check(c)
    _check(c, y_dtype="f32")


def test_no_user_rows_and_no_item_rows():
    _check(synth.lincomp_case(2, 3, 0, 64, 64, 16, seed=50, name="nu0"))
    _check(synth.lincomp_case(2, 3, 64, 0, 64, 16, seed=51, name="ni0"))


def test_integer_inputs_exact_f32():
    c = synth.lincomp_case(3, 4, 256, 256, 256, 64, x_dist=("int", -3, 3), w_dist=("int", -2, 2),
                           seed=52, name="lc_int")
    Y = _run(c, "f32")
    pairs = [(r, cc) for r in range(3) for cc in range(4)]
    ref = oracle.lincomp_case(c, pairs, bound=False)
    assert np.array_equal(np.stack([Y[r, cc] for r, cc in pairs]), ref)


def test_no_dedup_mode_matches_dedup():
    import recsys_linear_layers_amd as ll
    c = synth.lincomp_case(3, 5, 256, 256, 256, 64, seed=53, name="nodedup")
    a = _run(c)
    b = _check(c, flags=ll.LL_LINCOMP_NO_DEDUP)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Nu,Ni,D,Mo", [(256, 256, 256, 64), (40, 24, 72, 24), (0, 64, 64, 16)])
def test_stacked_input_matches_oracle_and_dedup(Nu, Ni, D, Mo):
    # Per-candidate user rows: no sharing, every candidate computes both sums
    # in the dedup path's order, so the results must be bit-identical.
    c = synth.lincomp_case(3, 5, Nu, Ni, D, Mo, seed=60 + Nu + Ni, name=f"stacked{Nu}_{Ni}_{D}_{Mo}")
    a = _run(c)
    b = _check(c, stacked=True)
    assert np.array_equal(a, b)
    _check(c, y_dtype="f32", stacked=True)


def test_full_workload_stacked_sampled_candidates():
    c = synth.lincomp_workload("lincomp_256x128")
    rng = np.random.default_rng(1)
    pairs = [(0, 0), (c.R - 1, c.C - 1)]
    pairs += [(int(r), int(k)) for r, k in zip(rng.integers(0, c.R, 16), rng.integers(0, c.C, 16))]
    _check(c, pairs, stacked=True)


def test_full_workload_sampled_candidates():
    c = synth.lincomp_workload("lincomp_256x128")
    rng = np.random.default_rng(0)
    pairs = [(0, 0), (c.R - 1, c.C - 1), (0, c.C - 1), (c.R - 1, 0)]
    pairs += [(int(r), int(k)) for r, k in zip(rng.integers(0, c.R, 40), rng.integers(0, c.C, 40))]
    _check(c, pairs)
