"""Ragged linear compression (variable candidates per request, flat candidate
axis with request offsets) on the GPU against the per-candidate fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import lincomp_operands, ragged_operands, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _run(case, y_dtype="bf16", flags=0):
    import torch
    import recsys_linear_layers_amd as ll
    user, item, W, offsets = ragged_operands(case)
    dt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    Y = torch.full((case.Ctot, case.Mo, case.D), float("nan"), dtype=dt, device="cuda")
    ll.lincomp_ragged(user, item, W, offsets, out=Y, flags=flags)
    torch.cuda.synchronize()
    return to_f64(Y)


def _check(case, gs=None, y_dtype="bf16", flags=0):
    Y = _run(case, y_dtype, flags)
    gs = list(range(case.Ctot)) if gs is None else gs
    pairs = [(case.request_of(g), g) for g in gs]
    ref, S = oracle.lincomp_naive(case.dims, case.user, case.item, case.W, case.strides, pairs)
    acceptance.assert_close(Y[gs], ref, S, y_dtype, case.name)
    return Y


@pytest.mark.parametrize("lengths", [[3, 0, 1, 5, 0, 0, 2], [0, 4, 0], [1], [0, 0, 6, 0, 0]])
def test_small_with_empty_requests(lengths):
    c = synth.lincomp_ragged_case(lengths, seed=70, sub=len(lengths), name=f"ragged{lengths}")
    a = _check(c)
    _check(c, y_dtype="f32")
    # every request's user block either once or per candidate: same sums, same order
    import recsys_linear_layers_amd as ll
    b = _run(c, flags=ll.LL_LINCOMP_NO_DEDUP)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Nu,Ni,D,Mo", [(40, 24, 72, 24), (0, 64, 64, 16), (64, 0, 64, 16), (8, 200, 264, 72)])
def test_ragged_dims(Nu, Ni, D, Mo):
    lengths = synth.ragged_lengths(9, 4.0, 0.8, seed=71, sub=Nu + Ni, lo=0, hi=12)
    c = synth.lincomp_ragged_case(lengths, Nu, Ni, D, Mo, seed=72, sub=Nu + Ni, name=f"ragged_{Nu}_{Ni}_{D}_{Mo}")
    _check(c)


def test_equal_lengths_match_per_request_path():
    # With C candidates for every request the ragged path and the per-request
    # path compute the same sums in the same order: bit-identical results.
    import torch
    import recsys_linear_layers_amd as ll
    reg = synth.lincomp_case(4, 6, 256, 256, 256, 64, seed=73, name="reg")
    user, item, W = lincomp_operands(reg)
    Y = torch.empty((4, 6, 64, 256), dtype=torch.bfloat16, device="cuda")
    ll.lincomp(user, item, W, out=Y)
    offsets = torch.arange(0, 25, 6, dtype=torch.int64, device="cuda")
    Yr = ll.lincomp_ragged(user, item.reshape(24, 256, 256), W, offsets)
    torch.cuda.synchronize()
    assert torch.equal(Y.reshape(24, 64, 256).view(torch.int16), Yr.view(torch.int16))


def test_many_short_requests():
    # more requests than workgroups, most ranges cross several requests
    lengths = synth.ragged_lengths(700, 3.0, 0.7, seed=74, lo=0, hi=9)
    c = synth.lincomp_ragged_case(lengths, 64, 64, 64, 16, seed=75, name="ragged_many")
    _check(c)


def test_full_workload_sampled_candidates():
    c = synth.lincomp_ragged_workload("lincomp_ragged_256")
    rng = np.random.default_rng(2)
    # first and last candidate of a few requests (range and request boundaries) plus random ones
    gs = [0, c.Ctot - 1]
    for r in (0, 1, 77, 128, 254, 255):
        gs += [int(c.offsets[r]), int(c.offsets[r + 1]) - 1]
    gs += [int(g) for g in rng.integers(0, c.Ctot, 40)]
    _check(c, sorted(set(gs)))
