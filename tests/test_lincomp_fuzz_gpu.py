"""Seeded random linear-compression cases on the GPU against the per-candidate
fp64 oracle: request and candidate counts, user / item row counts (user rows
may be absent), embedding width and output rows drawn at random, with bf16 or
fp32 Y, the user-once and the repeated-user modes, random ragged
request-length mixes (empty requests included), and the fused epilogue (bias
and activation) drawn at random too.  Reproducible per index."""
import numpy as np
import pytest

import oracle
import synth
from helpers import lincomp_operands, ragged_operands, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu

N_CASES = 40


def _dims(rng):
    def m8(lo, hi):
        return 8 * int(rng.integers(lo, hi + 1))
    Nu = 0 if rng.random() < 0.15 else m8(1, 40)
    Ni = m8(1, 40)
    D = m8(1, 40)
    Mo = m8(1, 17)
    return Nu, Ni, D, Mo


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_dense(i):
    import torch
    import recsys_linear_layers_amd as ll
    rng = np.random.default_rng(3000 + i)
    R, C = int(rng.integers(1, 7)), int(rng.integers(1, 10))
    Nu, Ni, D, Mo = _dims(rng)
    y = str(rng.choice(["bf16", "f32"]))
    flags = ll.LL_LINCOMP_NO_DEDUP if rng.random() < 0.3 else 0
    c = synth.lincomp_case(R, C, Nu, Ni, D, Mo, seed=4000 + i, name=f"fuzz{i}")
    user, item, W = lincomp_operands(c)
    Y = torch.full((R, C, Mo, D), float("nan"), dtype=torch.bfloat16 if y == "bf16" else torch.float32,
                   device="cuda")
    ll.lincomp(user, item, W, out=Y, flags=flags)
    torch.cuda.synchronize()
    got = to_f64(Y)
    pairs = [(r, cc) for r in range(R) for cc in range(C)]
    ref, S = oracle.lincomp_case(c, pairs)
    acceptance.assert_close(np.stack([got[r, cc] for r, cc in pairs]), ref, S, y,
                            f"case {i}: R={R} C={C} Nu={Nu} Ni={Ni} D={D} Mo={Mo} y={y} flags={flags}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_ragged(i):
    import torch
    import recsys_linear_layers_amd as ll
    rng = np.random.default_rng(5000 + i)
    R = int(rng.integers(1, 9))
    lengths = [0 if rng.random() < 0.25 else int(rng.integers(1, 8)) for _ in range(R)]
    Nu, Ni, D, Mo = _dims(rng)
    y = str(rng.choice(["bf16", "f32"]))
    c = synth.lincomp_ragged_case(lengths, Nu, Ni, D, Mo, seed=6000 + i, name=f"rfuzz{i}")
    user, item, W, offsets = ragged_operands(c)
    Y = torch.full((max(c.Ctot, 1), Mo, D), float("nan"), dtype=torch.bfloat16 if y == "bf16" else torch.float32,
                   device="cuda")[:c.Ctot]
    ll.lincomp_ragged(user, item, W, offsets, out=Y)
    torch.cuda.synchronize()
    if c.Ctot == 0:
        return
    got = to_f64(Y)
    gs = list(range(c.Ctot))
    pairs = [(c.request_of(g), g) for g in gs]
    ref, S = oracle.lincomp_naive(c.dims, c.user, c.item, c.W, c.strides, pairs)
    acceptance.assert_close(got, ref, S, y, f"ragged case {i}: lengths={lengths} Nu={Nu} Ni={Ni} D={D} Mo={Mo} y={y}")


N_EPI = 24


def _epilogue(rng, Mo):
    import torch
    act = rng.choice([None, "relu", "gelu", "silu"])
    if act is None or rng.random() < 0.7:
        b = (rng.standard_normal(Mo) * 0.5).astype(np.float32)
        return act, b, torch.from_numpy(b).cuda()
    return act, None, None


@pytest.mark.parametrize("i", range(N_EPI))
def test_random_dense_epilogue(i):
    import torch
    import recsys_linear_layers_amd as ll
    rng = np.random.default_rng(8000 + i)
    R, C = int(rng.integers(1, 7)), int(rng.integers(1, 10))
    Nu, Ni, D, Mo = _dims(rng)
    y = str(rng.choice(["bf16", "f32"]))
    flags = ll.LL_LINCOMP_NO_DEDUP if rng.random() < 0.3 else 0
    act, b, bt = _epilogue(rng, Mo)
    c = synth.lincomp_case(R, C, Nu, Ni, D, Mo, seed=9000 + i, name=f"efuzz{i}")
    user, item, W = lincomp_operands(c)
    Y = torch.full((R, C, Mo, D), float("nan"), dtype=torch.bfloat16 if y == "bf16" else torch.float32,
                   device="cuda")
    ll.lincomp(user, item, W, out=Y, flags=flags, bias=bt, act=act)
    torch.cuda.synchronize()
    got = to_f64(Y)
    pairs = [(r, cc) for r in range(R) for cc in range(C)]
    ref, S = oracle.lincomp_case(c, pairs)
    ref, S = oracle.lincomp_epilogue(ref, S, b, act)
    acceptance.assert_close(np.stack([got[r, cc] for r, cc in pairs]), ref, S, y,
                            f"epilogue case {i}: R={R} C={C} Nu={Nu} Ni={Ni} D={D} Mo={Mo} y={y} flags={flags} "
                            f"bias={b is not None} act={act}", act=act)


@pytest.mark.parametrize("i", range(N_EPI))
def test_random_ragged_epilogue(i):
    import torch
    import recsys_linear_layers_amd as ll
    rng = np.random.default_rng(8500 + i)
    R = int(rng.integers(1, 9))
    lengths = [0 if rng.random() < 0.25 else int(rng.integers(1, 8)) for _ in range(R)]
    Nu, Ni, D, Mo = _dims(rng)
    y = str(rng.choice(["bf16", "f32"]))
    act, b, bt = _epilogue(rng, Mo)
    c = synth.lincomp_ragged_case(lengths, Nu, Ni, D, Mo, seed=9500 + i, name=f"erfuzz{i}")
    user, item, W, offsets = ragged_operands(c)
    Y = torch.full((max(c.Ctot, 1), Mo, D), float("nan"), dtype=torch.bfloat16 if y == "bf16" else torch.float32,
                   device="cuda")[:c.Ctot]
    ll.lincomp_ragged(user, item, W, offsets, out=Y, bias=bt, act=act)
    torch.cuda.synchronize()
    if c.Ctot == 0:
        return
    pairs = [(c.request_of(g), g) for g in range(c.Ctot)]
    ref, S = oracle.lincomp_naive(c.dims, c.user, c.item, c.W, c.strides, pairs)
    ref, S = oracle.lincomp_epilogue(ref, S, b, act)
    acceptance.assert_close(to_f64(Y), ref, S, y, f"ragged epilogue case {i}: lengths={lengths} Nu={Nu} Ni={Ni} "
                            f"D={D} Mo={Mo} y={y} bias={b is not None} act={act}", act=act)
