"""Launches captured in a HIP graph replay the eager results bit for bit.

The library's run calls launch kernels only (no allocation, no memset), so a
caller can capture them on its stream.  Each graph is replayed several times
with unrelated eager work and synchronisations in between, and every replay is
compared with the eager result of the same call (same kernels, same order of
summation, so the results are identical)."""
import pytest

import synth
from synth.device import gemm_operands, lincomp_operands

pytestmark = pytest.mark.gpu


def _ll():
    import recsys_linear_layers_amd as ll
    return ll


def _replay_check(run, out, replays=3):
    """run() launches on torch's current stream and writes `out`."""
    import torch
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream before capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    x = torch.randn(512, 512, device="cuda")
    for i in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), eager.view(torch.uint8)), f"replay {i} differs"
        x = x @ x.t() / 512.0          # unrelated eager work between replays
        torch.cuda.synchronize()


def _gemm_case_run(case, flags=0, bias=None, act=None):
    import torch
    ll = _ll()
    A, B = gemm_operands(case)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[case.out_dtype]
    C = torch.empty((case.M, case.N), dtype=dt, device="cuda")
    epi = ll.ACTIVATIONS[act] | (ll.LL_EPI_BIAS if bias is not None else 0)
    plan = ll.plan_for(A, B, C, flags, epi)   # plan and workspace made before capture
    return plan, (lambda: plan.run(A, B, C, bias=bias)), C


def test_gemm_graph_replay():
    plan, run, C = _gemm_case_run(synth.gemm_case(1000, 1500, 700, seed=31, dist=("normal", 0.0, 1.0),
                                                  out_dtype="bf16"))
    _replay_check(run, C)


def test_gemm_split_k_graph_replay():
    # two kernels per call: partial tiles, then the ordered reduce
    plan, run, C = _gemm_case_run(synth.gemm_case(128, 2048, 8192, seed=32, out_dtype="f32"))
    assert "splitk=1 " not in plan.describe()
    _replay_check(run, C)


def test_gemm_packed_graph_replay():
    # odd leading dimensions: pack kernels run before the GEMM in the same call
    plan, run, C = _gemm_case_run(synth.gemm_case(777, 555, 333, seed=33, b_col_major=True, lda=335, ldb=337,
                                                  out_dtype="f32"))
    assert "packA=1" in plan.describe() and "packB=1" in plan.describe()
    _replay_check(run, C)


def test_gemm_fused_epilogue_graph_replay():
    import torch
    bias = torch.linspace(-1.0, 1.0, 1500, dtype=torch.float32, device="cuda")
    plan, run, C = _gemm_case_run(synth.gemm_case(1000, 1500, 700, seed=34, out_dtype="bf16"), bias=bias,
                                  act="gelu")
    _replay_check(run, C)


def test_lincomp_graph_replay():
    import torch
    ll = _ll()
    c = synth.lincomp_case(8, 5, 256, 256, 256, 64, seed=35)
    user, item, W = lincomp_operands(c)
    Y = torch.empty((c.R, c.C, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    _replay_check(lambda: ll.lincomp(user, item, W, out=Y), Y)


def test_hand_ordered_kind_graph_replay():
    # 5100 x 5120 selects the hand-ordered 256x256 kind: 400 work items on 256
    # workgroups (second items after the barrier that guards the staged C
    # image), a ragged last tile row (direct stores) beside staged tiles
    plan, run, C = _gemm_case_run(synth.gemm_case(5100, 5120, 256, seed=36, dist=("normal", 0.0, 1.0),
                                                  out_dtype="bf16"))
    assert "kernel=KIND_SQ4_HO " in plan.describe(), plan.describe()
    _replay_check(run, C)


def test_hand_ordered_kind_fused_graph_replay():
    import torch
    bias = torch.linspace(-2.0, 2.0, 5120, dtype=torch.float32, device="cuda")
    plan, run, C = _gemm_case_run(synth.gemm_case(5100, 5120, 256, seed=37, dist=("normal", 0.0, 1.0),
                                                  out_dtype="bf16"), bias=bias, act="silu")
    assert "kernel=KIND_SQ4_HO " in plan.describe(), plan.describe()
    _replay_check(run, C)


def test_lincomp_epilogue_graph_replay():
    import torch
    ll = _ll()
    c = synth.lincomp_case(8, 5, 256, 256, 256, 64, seed=38)
    user, item, W = lincomp_operands(c)
    bias = torch.linspace(-1.0, 1.0, 64, dtype=torch.float32, device="cuda")
    Y = torch.empty((c.R, c.C, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    _replay_check(lambda: ll.lincomp(user, item, W, out=Y, bias=bias, act="gelu"), Y)


@pytest.mark.parametrize("b_col", [False, True])
def test_hand_ordered_round_barrier_tail_prefetch_graph_replay(b_col, monkeypatch):
    # 4352 x 4096 x 2048 with the round barrier and the B prefetch forced on:
    # four kernels per call (counter clear, the GEMM, whose last round of 16
    # tiles is split two ways along K, and the ordered tail reduce); B
    # N-contiguous, or K-contiguous (the kind's variant for it)
    ll = _ll()
    ll._plans.clear()
    monkeypatch.setenv("LL_GEMM_KIND", "KIND_SQ4_HO")
    monkeypatch.setenv("LL_GEMM_ROUND_SYNC", "1")
    monkeypatch.setenv("LL_GEMM_PREFETCH_B", "1")
    try:
        plan, run, C = _gemm_case_run(synth.gemm_case(4352, 4096, 2048, seed=39 + b_col, dist=("normal", 0.0, 1.0),
                                                      out_dtype="bf16", b_col_major=b_col))
    finally:
        for v in ("LL_GEMM_KIND", "LL_GEMM_ROUND_SYNC", "LL_GEMM_PREFETCH_B"):
            monkeypatch.delenv(v, raising=False)
    d = plan.describe()
    assert "round_sync=1" in d and "tail=16x2" in d and "prefetch_b=1" in d, d
    assert ("B:K-major" if b_col else "B:N-major") in d, d
    _replay_check(run, C)
    ll._plans.clear()
