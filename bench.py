"""Benchmark: bf16 GEMM TFLOP/s (fraction of dense MFMA peak) and
linear-compression requests/s (fraction of HBM bandwidth) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the library on the headline workload (default: the
4096^3 GEMM with bf16 output).  Inputs are seeded synthetic bf16 (the
``synth`` module), resident in HBM before timing starts.  W untimed warm-up
steps, then K timed steps between two device synchronisations; the kernel's
average duration comes from HIP events recorded around every launch on the
stream the library launches on.  Prints ONE JSON line.  The other
configurations are reported in the same line under "also".

CPU baseline: the fp64 oracle, timed on a bounded sample of the headline
workload (rows of C) on this host's cores; it is a reported baseline, not the
target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

GEMM_NAMES = {"gemm_4096", "ffn_up", "ffn_down", "edge", "skinny_splitk", "gemm_256", "gemm_4096_f16", "gemm_3000"}
# workloads also timed with the kind the plan would choose without its tile
# rules (the 192x256 tile-count rule on gemm_3000, the 256x256 rule on the
# others)
TILE_RULE_NAMES = {"gemm_3000": "KIND_WIDE_PC", "gemm_4096": "KIND_WIDE_PC", "ffn_up": "KIND_WIDE_PC",
                   "gemm_4096_f16": "KIND_WIDE_PC"}
LINCOMP_NAMES = {"lincomp_256x128"}
# The same workload given in the layer's original form: every candidate's
# stacked input [user rows; item rows] materialised (no reuse possible).
STACKED_NAMES = {"lincomp_256x128_stacked": "lincomp_256x128"}
# Ragged requests: 256 requests with a lognormal mix of candidate counts.
RAGGED_NAMES = {"lincomp_ragged_256"}
# FFN up-projection with its bias and GELU fused into the GEMM's epilogue,
# against the same GEMM followed by separate bias-add and GELU passes.
EPILOGUE_NAMES = {"ffn_up_bias_gelu": "ffn_up"}


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recsys_linear_layers_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_from_profiles(workload: str):
    """HBM bytes per launch recorded by the rocprofv3 counter runs in profiles/,
    or None if there is no record or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_hash:\s*(\w+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != _kernel_source_hash():
        return None
    return float(b.group(1))


def _log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _time_launches(fn, steps: int, warmup: int, stream):
    """Returns (wall ms per step, event-measured ms per step).

    The K timed steps are enqueued back to back between one pair of HIP
    events recorded on `stream` (the stream the library launches on), so the
    per-step figure is the kernels' average duration plus any gap between
    them; the host stays ahead of the device for kernels this long.
    """
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, start.elapsed_time(end) / steps


def bench_gemm(name: str, steps: int, warmup: int, force_kind: str | None = None):
    """force_kind: time the plan with this kernel kind instead of the plan's own
    choice (LL_GEMM_KIND, read when a plan is made; the forced plan is not kept)."""
    import torch
    import recsys_linear_layers_amd as ll
    import synth
    from synth.device import gemm_operands
    _log(f"{name}: generating inputs")
    case = synth.gemm_workload(name)
    A, B = gemm_operands(case)
    _log(f"{name}: timing" + (f" with {force_kind}" if force_kind else ""))
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[case.out_dtype]
    C = torch.empty((case.M, case.N), dtype=dt, device="cuda")
    if force_kind:
        os.environ["LL_GEMM_KIND"] = force_kind
        try:
            plan = ll.GemmPlan(ll.gemm_desc_for(A, B, C), A.device)
        finally:
            del os.environ["LL_GEMM_KIND"]
    else:
        plan = ll.plan_for(A, B, C)
    stream = torch.cuda.current_stream()
    wall, ev = _time_launches(lambda: plan.run(A, B, C, stream.cuda_stream), steps, warmup, stream)
    tflops = case.flops / (ev * 1e-3) / 1e12
    return dict(case=case, wall_ms=wall, kernel_ms=ev, tflops=tflops, plan=plan.describe())


def bench_lincomp(name: str, steps: int, warmup: int):
    import torch
    import recsys_linear_layers_amd as ll
    import synth
    from synth.device import lincomp_operands
    _log(f"{name}: generating inputs")
    c = synth.lincomp_workload(name)
    user, item, W = lincomp_operands(c)
    _log(f"{name}: timing")
    Y = torch.empty((c.R, c.C, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    wall, ev = _time_launches(lambda: ll.lincomp(user, item, W, out=Y), steps, warmup, stream)
    gbs = c.algorithmic_bytes / (ev * 1e-3) / 1e9
    return dict(case=c, wall_ms=wall, kernel_ms=ev, req_s=c.R / (ev * 1e-3), gbs=gbs,
                tflops=c.flops / (ev * 1e-3) / 1e12)


def bench_lincomp_stacked(name: str, steps: int, warmup: int):
    """Times linear compression on the materialised stacked input X
    [R][C][Nu+Ni][D] and, on the same data, the user-once form; reports the
    ratio of the two (the speedup of computing the user block once)."""
    import torch
    import recsys_linear_layers_amd as ll
    import synth
    from synth.device import lincomp_operands
    c = synth.lincomp_workload(STACKED_NAMES[name])
    user, item, W = lincomp_operands(c)
    X = torch.cat([user[:, None].expand(c.R, c.C, c.Nu, c.D), item], dim=2).contiguous()
    Y = torch.empty((c.R, c.C, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    _log(f"{name}: timing the stacked input")
    wall, ev = _time_launches(lambda: ll.lincomp_stacked(X, W, c.Nu, out=Y), steps, warmup, stream)
    _log(f"{name}: timing the user-once form on the same data")
    _, ev_dedup = _time_launches(lambda: ll.lincomp(user, item, W, out=Y), steps, warmup, stream)
    stacked_bytes = X.numel() * 2 + W.numel() * 2 + Y.numel() * 2
    return dict(case=c, wall_ms=wall, kernel_ms=ev, req_s=c.R / (ev * 1e-3),
                gbs=stacked_bytes / (ev * 1e-3) / 1e9, stacked_bytes=stacked_bytes,
                dedup_ms=ev_dedup, speedup=ev / ev_dedup)


def bench_lincomp_ragged(name: str, steps: int, warmup: int):
    import torch
    import recsys_linear_layers_amd as ll
    import synth
    from synth.device import ragged_operands
    _log(f"{name}: generating inputs")
    c = synth.lincomp_ragged_workload(name)
    user, item, W, offsets = ragged_operands(c)
    Y = torch.empty((c.Ctot, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    _log(f"{name}: timing")
    wall, ev = _time_launches(lambda: ll.lincomp_ragged(user, item, W, offsets, out=Y), steps, warmup, stream)
    gbs = c.algorithmic_bytes / (ev * 1e-3) / 1e9
    return dict(case=c, wall_ms=wall, kernel_ms=ev, req_s=c.R / (ev * 1e-3), gbs=gbs)


def bench_gemm_epilogue(name: str, steps: int, warmup: int):
    import torch
    import recsys_linear_layers_amd as ll
    import synth
    from synth.device import gemm_operands
    case = synth.gemm_workload(EPILOGUE_NAMES[name])
    A, B = gemm_operands(case)
    bias = torch.randn(case.N, dtype=torch.float32, device="cuda") * 0.5
    C = torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    fused = ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.LL_EPI_GELU)
    plain = ll.plan_for(A, B, C)
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    _log(f"{name}: timing the fused epilogue")
    _, ev_fused = _time_launches(lambda: fused.run(A, B, C, h, bias=bias), steps, warmup, stream)
    b16 = bias.to(torch.bfloat16)

    def unfused():
        plain.run(A, B, C, h)
        torch.nn.functional.gelu(C + b16)

    _log(f"{name}: timing GEMM + separate bias and GELU passes")
    _, ev_unfused = _time_launches(unfused, steps, warmup, stream)
    return dict(case=case, fused_ms=ev_fused, unfused_ms=ev_unfused, plan=fused.describe(),
                tflops=case.flops / (ev_fused * 1e-3) / 1e12)


def cpu_baseline_gemm(name: str, target_s: float = 12.0):
    """The oracle on the first rows of C, sized to about target_s of CPU time."""
    import oracle
    import synth
    case = synth.gemm_workload(name)
    rows, dt = 1, 0.0
    while rows < case.M:
        t0 = time.perf_counter()
        oracle.gemm_case(case, rows=(0, rows), bound=False)
        dt = time.perf_counter() - t0
        if dt > 0.5:
            break
        rows *= 2
    rows = int(max(1, min(case.M, rows * target_s / max(dt, 1e-6))))
    t0 = time.perf_counter()
    oracle.gemm_case(case, rows=(0, rows), bound=False)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * case.N * case.K
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=oracle.get_threads(), kind="oracle",
                sample=f"fp64 oracle, rows 0..{rows - 1} of C ({rows}x{case.N}x{case.K}), {dt:.1f} s")


def cpu_baseline_lincomp(name: str, target_s: float = 12.0):
    import oracle
    import synth
    c = synth.lincomp_workload(name)
    n, dt = 1, 0.0
    while n < c.R * c.C:
        t0 = time.perf_counter()
        oracle.lincomp_case(c, [(i // c.C, i % c.C) for i in range(n)], bound=False)
        dt = time.perf_counter() - t0
        if dt > 0.5:
            break
        n *= 2
    n = int(max(1, min(c.R * c.C, n * target_s / max(dt, 1e-6))))
    pairs = [(i // c.C, i % c.C) for i in range(n)]
    t0 = time.perf_counter()
    oracle.lincomp_case(c, pairs, bound=False)
    dt = time.perf_counter() - t0
    # requests/s at this candidate rate
    return dict(value=(n / c.C) / dt, unit="requests/s", cores=oracle.get_threads(), kind="oracle",
                sample=f"fp64 per-candidate oracle, first {n} candidates, {dt:.1f} s")


def vendor_context(steps: int, warmup: int):
    """torch.matmul on the GEMM workloads' shapes, operands of the same types
    and scales drawn on the device, timed like the library (same warm-up and
    step counts, one event pair around the timed calls)."""
    import torch
    import synth
    out = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    for name in ["gemm_4096", "ffn_up", "ffn_down", "gemm_3000", "gemm_4096_f16", "skinny_splitk"]:
        M, N, K, kw = synth.GEMM_WORKLOADS[name]
        in_t = {"bf16": torch.bfloat16, "f16": torch.float16}[kw.get("in_dtype", "bf16")]
        def draw(rows, cols, dist):
            if dist[0] == "uniform":
                return (torch.rand(rows, cols, device="cuda", generator=gen) * (dist[2] - dist[1]) + dist[1]).to(in_t)
            return (torch.randn(rows, cols, device="cuda", generator=gen) * dist[2] + dist[1]).to(in_t)
        A = draw(M, K, kw["dist"])
        B = draw(K, N, kw.get("b_dist") or kw["dist"])
        # torch.matmul writes C in its inputs' type: an fp32-output workload is
        # timed with a bf16/fp16 C (noted in the result)
        C = torch.empty(M, N, device="cuda", dtype=in_t)
        _log(f"vendor context: {name}")
        _, ev = _time_launches(lambda: torch.matmul(A, B, out=C), steps, warmup, torch.cuda.current_stream())
        out.append(dict(workload=name, ms=round(ev, 4), tflops=round(2.0 * M * N * K / (ev * 1e-3) / 1e12, 1),
                        c_dtype=str(C.dtype).replace("torch.", ""), library_c_dtype=kw.get("out_dtype", "f32")))
        del A, B, C
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Short kernels need tens of milliseconds of back-to-back work before the
    # clocks settle: the 4096^3 GEMM (~0.12 ms per call) measured ~20% low
    # after 5 warm-up calls, ~9% low after 50, and within 1% of its steady
    # rate after 300 or 1000.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="gemm_4096",
                    choices=sorted(GEMM_NAMES | LINCOMP_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="time only the headline workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, --steps times "
                         "(calibrates the HBM byte counters of a profiler run); prints its own line")
    ap.add_argument("--vendor-context", action="store_true",
                    help="time torch.matmul (the vendor GEMM) on the GEMM workloads' shapes instead, for context")
    ap.add_argument("--stream-probe-mib", type=int, default=0,
                    help="only run a streaming reduction that reads 4x and writes 1x this many MiB "
                         "(the read/write mix of linear compression), --steps times; prints its own line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream()
        wall, ev = _time_launches(lambda: dst.copy_(src), args.steps, args.warmup, stream)
        print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": round(ev, 4),
                          "GB/s": round(2 * n / (ev * 1e-3) / 1e9, 1)}))
        return

    if args.stream_probe_mib:
        # out[i] = x[0][i] + x[1][i] + x[2][i] + x[3][i]: 4 bytes read per byte
        # written, a plain streaming pass with no reuse.
        n = (args.stream_probe_mib << 20) // 4
        x = torch.ones((4, n), dtype=torch.float32, device="cuda")
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        wall, ev = _time_launches(lambda: torch.sum(x, dim=0, out=y), args.steps, args.warmup, stream)
        rd, wr = 16 * n, 4 * n
        print(json.dumps({"probe": "stream 4 reads : 1 write", "bytes_read": rd, "bytes_written": wr,
                          "ms": round(ev, 4), "GB/s": round((rd + wr) / (ev * 1e-3) / 1e9, 1)}))
        return

    if args.vendor_context:
        print(json.dumps({"probe": "vendor GEMM (torch.matmul), context only", "steps": args.steps,
                          "warmup": args.warmup, "results": vendor_context(args.steps, args.warmup)}))
        return

    head = args.workload
    rule_context = {}
    if head in LINCOMP_NAMES:
        r = bench_lincomp(head, args.steps, args.warmup)
        c = r["case"]
        metric, unit, value = "linear-compression requests/s", "requests/s", r["req_s"]
        roof = dict(bound="hbm", achieved=r["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=r["gbs"] / PEAK_HBM_GBS, traffic=_traffic_from_profiles(head))
        config = dict(workload=head, requests=c.R, candidates_per_request=c.C, user_rows=c.Nu,
                      item_rows=c.Ni, dim=c.D, out_rows=c.Mo, y_dtype="bf16",
                      algorithmic_bytes=c.algorithmic_bytes)
        plan = ("one persistent launch: per request the user block's product once, kept in registers "
                "and reused as every candidate's starting sums; 4 loading + 4 computing waves")
    else:
        r = bench_gemm(head, args.steps, args.warmup)
        c = r["case"]
        metric, unit, value = "bf16 GEMM TFLOP/s", "TFLOP/s", r["tflops"]
        roof = dict(bound="mfma", achieved=r["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=r["tflops"] / PEAK_BF16_TFLOPS, traffic=_traffic_from_profiles(head))
        config = dict(workload=head, M=c.M, N=c.N, K=c.K, a_layout="row-major",
                      b_layout="column-major" if c.sbk == 1 else "row-major",
                      c_dtype=c.out_dtype, flops=c.flops)
        plan = r["plan"]
        if head in TILE_RULE_NAMES:
            y = bench_gemm(head, args.steps, args.warmup, force_kind=TILE_RULE_NAMES[head])
            rule_context = dict(without_rule_ms=round(y["kernel_ms"], 4), without_rule_tflops=round(y["tflops"], 1),
                                tile_rule_speedup=round(y["kernel_ms"] / r["kernel_ms"], 3),
                                plan_without_rule=y["plan"])

    also = []
    if not args.no_also:
        for name in ["ffn_up", "ffn_down", "ffn_up_bias_gelu", "lincomp_256x128", "lincomp_256x128_stacked",
                     "lincomp_ragged_256",
                     "edge", "skinny_splitk", "gemm_3000", "gemm_4096_f16", "gemm_4096"]:
            if name == head:
                continue
            torch.cuda.empty_cache()
            if name in TILE_RULE_NAMES:
                x = bench_gemm(name, args.steps, args.warmup)
                y = bench_gemm(name, args.steps, args.warmup, force_kind=TILE_RULE_NAMES[name])
                also.append(dict(workload=name, ms=round(x["kernel_ms"], 4), value=round(x["tflops"], 1),
                                 unit="TFLOP/s", mfma_frac=round(x["tflops"] / PEAK_BF16_TFLOPS, 4),
                                 without_rule_ms=round(y["kernel_ms"], 4),
                                 tile_rule_speedup=round(y["kernel_ms"] / x["kernel_ms"], 3), plan=x["plan"],
                                 plan_without_rule=y["plan"]))
            elif name in EPILOGUE_NAMES:
                x = bench_gemm_epilogue(name, args.steps, args.warmup)
                also.append(dict(workload=name, ms=round(x["fused_ms"], 4), value=round(x["tflops"], 1),
                                 unit="TFLOP/s", mfma_frac=round(x["tflops"] / PEAK_BF16_TFLOPS, 4),
                                 unfused_ms=round(x["unfused_ms"], 4),
                                 fused_speedup=round(x["unfused_ms"] / x["fused_ms"], 3), plan=x["plan"]))
            elif name in RAGGED_NAMES:
                x = bench_lincomp_ragged(name, args.steps, args.warmup)
                c = x["case"]
                also.append(dict(workload=name, ms=round(x["kernel_ms"], 4), value=round(x["req_s"], 1),
                                 unit="requests/s", candidates=c.Ctot,
                                 candidates_per_request=[int(c.lengths.min()), round(float(c.lengths.mean()), 1),
                                                         int(c.lengths.max())],
                                 hbm_gbs=round(x["gbs"], 1), hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4)))
            elif name in STACKED_NAMES:
                x = bench_lincomp_stacked(name, args.steps, args.warmup)
                also.append(dict(workload=name, ms=round(x["kernel_ms"], 4), value=round(x["req_s"], 1),
                                 unit="requests/s", hbm_gbs=round(x["gbs"], 1),
                                 hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4), bytes=x["stacked_bytes"],
                                 user_once_ms=round(x["dedup_ms"], 4),
                                 user_once_speedup=round(x["speedup"], 3)))
            elif name in LINCOMP_NAMES:
                x = bench_lincomp(name, args.steps, args.warmup)
                also.append(dict(workload=name, ms=round(x["kernel_ms"], 4), value=round(x["req_s"], 1),
                                 unit="requests/s", hbm_gbs=round(x["gbs"], 1),
                                 hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4)))
            else:
                x = bench_gemm(name, args.steps, args.warmup)
                also.append(dict(workload=name, ms=round(x["kernel_ms"], 4), value=round(x["tflops"], 1),
                                 unit="TFLOP/s", mfma_frac=round(x["tflops"] / PEAK_BF16_TFLOPS, 4),
                                 plan=x["plan"]))
            del x

    cpu = None
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        cpu = cpu_baseline_lincomp(head) if head in LINCOMP_NAMES else cpu_baseline_gemm(head)

    out = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["wall_ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": config, "roofline": roof, "cpu_baseline": cpu,
        "kernel_ms": round(r["kernel_ms"], 4), "plan": plan, **rule_context, "also": also,
        "kernel_source_hash": _kernel_source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
