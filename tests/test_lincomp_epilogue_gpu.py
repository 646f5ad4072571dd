"""Linear compression with its fused epilogue (a per-compressed-row fp32 bias,
then ReLU / GELU / SiLU on the fp32 sums before they are rounded) on the GPU
against the per-candidate fp64 oracle followed by the oracle's epilogue."""
import numpy as np
import pytest

import oracle
import synth
from helpers import lincomp_operands, ragged_operands, to_f64
from oracle import acceptance

pytestmark = pytest.mark.gpu


def _bias(Mo, seed, scale=0.5):
    import torch
    b = (np.random.default_rng(seed).standard_normal(Mo) * scale).astype(np.float32)
    return b, torch.from_numpy(b).cuda()


def _check(case, act, with_bias=True, y_dtype="bf16", flags=0, stacked=False, pairs=None):
    import torch
    import recsys_linear_layers_amd as ll
    R, C, D, Mo, Nu = case.R, case.C, case.D, case.Mo, case.Nu
    user, item, W = lincomp_operands(case)
    b, bt = _bias(Mo, Mo + D + Nu) if with_bias else (None, None)
    dt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    Y = torch.full((R, C, Mo, D), float("nan"), dtype=dt, device="cuda")
    if stacked:
        X = torch.cat([user[:, None].expand(R, C, Nu, D), item], dim=2).contiguous()
        ll.lincomp_stacked(X, W, Nu, out=Y, bias=bt, act=act)
    else:
        ll.lincomp(user, item, W, out=Y, flags=flags, bias=bt, act=act)
    torch.cuda.synchronize()
    got_all = to_f64(Y)
    pairs = pairs or [(r, c) for r in range(R) for c in range(C)]
    ref, S = oracle.lincomp_case(case, pairs)
    ref, S = oracle.lincomp_epilogue(ref, S, b, act)
    got = np.stack([got_all[r, c] for r, c in pairs])
    acceptance.assert_close(got, ref, S, y_dtype, f"{case.name} bias={with_bias} act={act}", act=act)
    return got_all


@pytest.mark.parametrize("act", [None, "relu", "gelu", "silu"])
@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
def test_small_workload(act, y_dtype):
    _check(synth.lincomp_workload("lincomp_small"), act, y_dtype=y_dtype)


@pytest.mark.parametrize("act", ["relu", "gelu", "silu"])
def test_activation_without_bias(act):
    _check(synth.lincomp_case(2, 3, 64, 64, 64, 16, seed=70, name="nobias"), act, with_bias=False)


@pytest.mark.parametrize("Nu,Ni,D,Mo", [(40, 24, 72, 24), (256, 64, 128, 64), (8, 200, 8, 8), (64, 64, 264, 72),
                                        (0, 64, 64, 16), (64, 0, 64, 16)])
def test_ragged_dims(Nu, Ni, D, Mo):
    c = synth.lincomp_case(2, 3, Nu, Ni, D, Mo, seed=71 + Nu + Ni, name=f"epi{Nu}_{Ni}_{D}_{Mo}")
    _check(c, "gelu")
    _check(c, "silu", y_dtype="f32")


def test_no_dedup_and_stacked_match_user_once():
    """The bias enters every path once per output: the user-once form, the
    no-dedup flag and the stacked input give bit-identical results."""
    import recsys_linear_layers_amd as ll
    c = synth.lincomp_case(3, 5, 256, 256, 256, 64, seed=72, name="epi_paths")
    a = _check(c, "gelu")
    b = _check(c, "gelu", flags=ll.LL_LINCOMP_NO_DEDUP)
    s = _check(c, "gelu", stacked=True)
    assert np.array_equal(a, b) and np.array_equal(a, s)


def test_ragged_requests():
    import torch
    import recsys_linear_layers_amd as ll
    lengths = [3, 0, 5, 1, 0, 7]
    c = synth.lincomp_ragged_case(lengths, Nu=64, Ni=64, D=128, Mo=32, seed=73, name="epi_ragged")
    user, item, W, offsets = ragged_operands(c)
    b, bt = _bias(c.Mo, 74)
    Y = torch.full((c.Ctot, c.Mo, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ll.lincomp_ragged(user, item, W, offsets, out=Y, bias=bt, act="silu")
    torch.cuda.synchronize()
    pairs = [(c.request_of(g), g) for g in range(c.Ctot)]
    ref, S = oracle.lincomp_naive(c.dims, c.user, c.item, c.W, c.strides, pairs)
    ref, S = oracle.lincomp_epilogue(ref, S, b, "silu")
    acceptance.assert_close(to_f64(Y), ref, S, "bf16", "ragged bias+silu", act="silu")


def test_full_workload_sampled_candidates():
    c = synth.lincomp_workload("lincomp_256x128")
    rng = np.random.default_rng(75)
    pairs = [(0, 0), (c.R - 1, c.C - 1)]
    pairs += [(int(r), int(k)) for r, k in zip(rng.integers(0, c.R, 24), rng.integers(0, c.C, 24))]
    _check(c, "gelu", pairs=pairs)


def test_errors():
    import torch
    import recsys_linear_layers_amd as ll
    c = synth.lincomp_case(2, 3, 64, 64, 64, 16, seed=76, name="epi_err")
    user, item, W = lincomp_operands(c)
    Y = torch.empty((2, 3, 16, 64), dtype=torch.bfloat16, device="cuda")
    _, bt = _bias(16, 77)
    d = ll.lincomp_desc_for(user, item, W, Y, 0, ll.LL_EPI_BIAS | ll.LL_EPI_RELU)
    with pytest.raises(ll.LLError):  # the plain entry point refuses an epilogue with a bias
        ll.lincomp_run(d, user.data_ptr(), item.data_ptr(), W.data_ptr(), Y.data_ptr(), 0, 0, 0)
    with pytest.raises(ll.LLError):  # null bias
        ll.lincomp_run_ex(d, user.data_ptr(), item.data_ptr(), W.data_ptr(), None, Y.data_ptr(), 0, 0, 0)
    with pytest.raises(ll.LLError):  # misaligned bias
        ll.lincomp_run_ex(d, user.data_ptr(), item.data_ptr(), W.data_ptr(), bt.data_ptr() + 4, Y.data_ptr(),
                          0, 0, 0)
    d.epilogue = 0x40
    with pytest.raises(ll.LLError):  # unknown activation
        ll.lincomp_run_ex(d, user.data_ptr(), item.data_ptr(), W.data_ptr(), None, Y.data_ptr(), 0, 0, 0)
