"""Benchmark: bf16 GEMM TFLOP/s (fraction of dense MFMA peak) and
linear-compression requests/s (fraction of HBM bandwidth) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the library on the headline workload (default: the
4096^3 GEMM with bf16 output).  Inputs are seeded synthetic bf16 (the
``synth`` module), resident in HBM before timing starts.  Every workload gets
W untimed warm-up calls, then K timed calls back to back between two device
synchronisations, with one pair of HIP events on the stream the library
launches on around the K calls: their mean is what throughput is computed
from.  A second pass of K calls, each bracketed by its own pair of events,
gives the median (per-call events put packets of their own between the
kernels, so that pass is not the one the mean comes from).
The other configurations (FFN shapes, linear compression and its variants,
edge and skinny shapes) run first and the headline last, so that the headline
is timed at the clocks the chip holds under sustained work rather than at
the clocks it ramps up from after idling through input generation.  Prints
ONE JSON line; linear compression, the second half of the metric, has its
own object ("lincomp") with its own roofline and CPU baseline.

CPU baseline: the fp64 oracle (the original, plain implementation) on this
host's cores, after all GPU timing: the whole headline problem, and per
configuration the whole problem where it takes seconds, or a bounded sample
(C3: a seeded 64-row strip plus the first and last rows, with the time for the
full shape extrapolated and labelled so).  It is a reported baseline, not the
target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

GEMM_NAMES = {"gemm_4096", "ffn_up", "ffn_down", "edge", "skinny_splitk", "gemm_256", "gemm_4096_f16", "gemm_3000",
              "gemm_4096_nt", "gemm_4096_tn"}
# workloads also timed with the kind the plan would choose without its tile
# rules (the 192x256 tile-count rule on gemm_3000, the 256x256 rule on the
# others)
TILE_RULE_NAMES = {"gemm_3000": "KIND_WIDE_PC", "gemm_4096": "KIND_WIDE_PC", "ffn_up": "KIND_WIDE_PC",
                   "gemm_4096_f16": "KIND_WIDE_PC", "gemm_4096_nt": "KIND_WIDE_PC",
                   "gemm_4096_tn": "KIND_WIDE_PC"}
LINCOMP_NAMES = {"lincomp_256x128"}
# The same workload given in the layer's original form: every candidate's
# stacked input [user rows; item rows] materialised (no reuse possible).
STACKED_NAMES = {"lincomp_256x128_stacked": "lincomp_256x128"}
# Ragged requests: 256 requests with a lognormal mix of candidate counts.
RAGGED_NAMES = {"lincomp_ragged_256"}
# FFN up-projection with its bias and GELU fused into the GEMM's epilogue,
# against the same GEMM followed by separate bias-add and GELU passes.
EPILOGUE_NAMES = {"ffn_up_bias_gelu": "ffn_up"}
# Linear compression with a per-compressed-row bias and GELU fused into its
# epilogue, against the plain layer followed by separate bias-add and GELU passes.
LC_EPILOGUE_NAMES = {"lincomp_256x128_bias_gelu": "lincomp_256x128"}


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
    """W untimed calls, then the timed region: K calls back to back between two
    device synchronisations, with one pair of HIP events recorded on `stream`
    (the stream the library launches on) around them and nothing else in the
    stream between the calls.  Then, in a second pass of K calls, a pair of
    events around each call gives the spread (median); those per-call events
    add their own packets between the kernels, so the mean comes from the
    first pass.  Returns dict(ms: mean per call over the timed region,
    wall_ms: host time per call across the timed region, median_ms and
    per_call_mean_ms: from the per-call pass)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    mean = e0.elapsed_time(e1) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return dict(wall_ms=wall, ms=mean, median_ms=statistics.median(per), per_call_mean_ms=statistics.fmean(per))


_CASES: dict = {}


def _case(name: str):
    """Host inputs of a workload, generated once and shared by its GPU leg and
    its CPU baseline (dropped by _drop_case)."""
    import synth
    if name not in _CASES:
        if name in LINCOMP_NAMES:
            _CASES[name] = synth.lincomp_workload(name)
        elif name in RAGGED_NAMES:
            _CASES[name] = synth.lincomp_ragged_workload(name)
        else:
            _CASES[name] = synth.gemm_workload(name)
    return _CASES[name]


def _drop_case(name: str) -> None:
    _CASES.pop(name, None)


# Every workload is prepared first (inputs copied to HBM, plans made), then
# all are timed back to back, so that no timed call follows a host-side pause.

def prep_gemm(name: str, force_kind: str | None = None) -> dict:
    """Device operands, output and plan of a GEMM workload.  force_kind: make the
    plan with this kernel kind instead of the plan's own choice (LL_GEMM_KIND,
    read when a plan is made; the forced plan is not cached)."""
    import torch
    import recsys_linear_layers_amd as ll
    from synth.device import gemm_operands
    _log(f"{name}: preparing inputs")
    case = _case(name)
    A, B = gemm_operands(case)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[case.out_dtype]
    C = torch.empty((case.M, case.N), dtype=dt, device="cuda")
    plans = {None: ll.plan_for(A, B, C)}
    if force_kind:
        os.environ["LL_GEMM_KIND"] = force_kind
        try:
            plans[force_kind] = ll.GemmPlan(ll.gemm_desc_for(A, B, C), A.device)
        finally:
            del os.environ["LL_GEMM_KIND"]
    return dict(case=case, A=A, B=B, C=C, plans=plans)


def time_gemm(p: dict, steps: int, warmup: int, kind: str | None = None) -> dict:
    import torch
    case, A, B, C, plan = p["case"], p["A"], p["B"], p["C"], p["plans"][kind]
    _log(f"{case.name}: timing" + (f" with {kind}" if kind else ""))
    stream = torch.cuda.current_stream()
    t = _time_launches(lambda: plan.run(A, B, C, stream.cuda_stream), steps, warmup, stream)
    return dict(case=case, wall_ms=t["wall_ms"], kernel_ms=t["ms"], median_ms=t["median_ms"],
                per_call_mean_ms=t["per_call_mean_ms"], tflops=case.flops / (t["ms"] * 1e-3) / 1e12, plan=plan.describe())


def prep_lincomp(name: str) -> dict:
    import torch
    from synth.device import lincomp_operands
    _log(f"{name}: preparing inputs")
    c = _case(name)
    user, item, W = lincomp_operands(c)
    Y = torch.empty((c.R, c.C, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    return dict(case=c, user=user, item=item, W=W, Y=Y)


def time_lincomp(p: dict, steps: int, warmup: int) -> dict:
    import torch
    import recsys_linear_layers_amd as ll
    c, user, item, W, Y = p["case"], p["user"], p["item"], p["W"], p["Y"]
    _log(f"{c.name}: timing")
    stream = torch.cuda.current_stream()
    t = _time_launches(lambda: ll.lincomp(user, item, W, out=Y), steps, warmup, stream)
    ev = t["ms"]
    return dict(case=c, wall_ms=t["wall_ms"], kernel_ms=ev, median_ms=t["median_ms"],
                per_call_mean_ms=t["per_call_mean_ms"], req_s=c.R / (ev * 1e-3),
                gbs=c.algorithmic_bytes / (ev * 1e-3) / 1e9, tflops=c.flops / (ev * 1e-3) / 1e12)


def prep_stacked(lc: dict) -> dict:
    """The workload's materialised stacked input X [R][C][Nu+Ni][D] (every
    candidate's [user rows; item rows]), built on the device from the
    user-once workload's operands."""
    import torch
    c = lc["case"]
    X = torch.cat([lc["user"][:, None].expand(c.R, c.C, c.Nu, c.D), lc["item"]], dim=2).contiguous()
    return dict(lc, X=X)


def time_stacked(p: dict, steps: int, warmup: int) -> dict:
    """Times linear compression on the stacked input and, on the same data, the
    user-once form; reports the ratio of the two (the speedup of computing the
    user block once)."""
    import torch
    import recsys_linear_layers_amd as ll
    c, X, W, Y = p["case"], p["X"], p["W"], p["Y"]
    stream = torch.cuda.current_stream()
    _log(f"{c.name}: timing the stacked input")
    t = _time_launches(lambda: ll.lincomp_stacked(X, W, c.Nu, out=Y), steps, warmup, stream)
    _log(f"{c.name}: timing the user-once form on the same data")
    td = _time_launches(lambda: ll.lincomp(p["user"], p["item"], W, out=Y), steps, warmup, stream)
    ev = t["ms"]
    stacked_bytes = X.numel() * 2 + W.numel() * 2 + Y.numel() * 2
    return dict(case=c, wall_ms=t["wall_ms"], kernel_ms=ev, median_ms=t["median_ms"], req_s=c.R / (ev * 1e-3),
                gbs=stacked_bytes / (ev * 1e-3) / 1e9, stacked_bytes=stacked_bytes,
                dedup_ms=td["ms"], speedup=ev / td["ms"])


def prep_ragged(name: str) -> dict:
    import torch
    from synth.device import ragged_operands
    _log(f"{name}: preparing inputs")
    c = _case(name)
    user, item, W, offsets = ragged_operands(c)
    Y = torch.empty((c.Ctot, c.Mo, c.D), dtype=torch.bfloat16, device="cuda")
    return dict(case=c, user=user, item=item, W=W, offsets=offsets, Y=Y)


def time_ragged(p: dict, steps: int, warmup: int) -> dict:
    import torch
    import recsys_linear_layers_amd as ll
    c = p["case"]
    stream = torch.cuda.current_stream()
    _log(f"{c.name}: timing")
    t = _time_launches(lambda: ll.lincomp_ragged(p["user"], p["item"], p["W"], p["offsets"], out=p["Y"]),
                       steps, warmup, stream)
    ev = t["ms"]
    return dict(case=c, wall_ms=t["wall_ms"], kernel_ms=ev, median_ms=t["median_ms"], req_s=c.R / (ev * 1e-3),
                gbs=c.algorithmic_bytes / (ev * 1e-3) / 1e9)


def prep_epilogue(g: dict) -> dict:
    """The FFN up-projection's operands with a per-column fp32 bias and GELU
    fused into the GEMM, against the plain GEMM followed by separate bias-add
    and GELU passes."""
    import torch
    import recsys_linear_layers_amd as ll
    A, B, case = g["A"], g["B"], g["case"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    bias = torch.randn(case.N, dtype=torch.float32, device="cuda", generator=gen) * 0.5
    C = torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda")
    return dict(case=case, A=A, B=B, C=C, bias=bias, b16=bias.to(torch.bfloat16),
                fused=ll.plan_for(A, B, C, 0, ll.LL_EPI_BIAS | ll.LL_EPI_GELU), plain=ll.plan_for(A, B, C))


def time_epilogue(p: dict, steps: int, warmup: int) -> dict:
    import torch
    A, B, C, case = p["A"], p["B"], p["C"], p["case"]
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream
    _log(f"{case.name}: timing the fused bias + GELU epilogue")
    tf = _time_launches(lambda: p["fused"].run(A, B, C, h, bias=p["bias"]), steps, warmup, stream)

    def unfused():
        p["plain"].run(A, B, C, h)
        torch.nn.functional.gelu(C + p["b16"])

    _log(f"{case.name}: timing GEMM + separate bias and GELU passes")
    tu = _time_launches(unfused, steps, warmup, stream)
    return dict(case=case, fused_ms=tf["ms"], median_ms=tf["median_ms"], unfused_ms=tu["ms"],
                plan=p["fused"].describe(), tflops=case.flops / (tf["ms"] * 1e-3) / 1e12)


def prep_lc_epilogue(lc: dict) -> dict:
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(43)
    c = lc["case"]
    bias = torch.randn(c.Mo, dtype=torch.float32, device="cuda", generator=gen) * 0.5
    return dict(lc, bias=bias, b16=bias.to(torch.bfloat16)[:, None])


def time_lc_epilogue(p: dict, steps: int, warmup: int) -> dict:
    import torch
    import recsys_linear_layers_amd as ll
    c, user, item, W, Y = p["case"], p["user"], p["item"], p["W"], p["Y"]
    stream = torch.cuda.current_stream()
    _log(f"{c.name}: timing the fused bias + GELU epilogue")
    tf = _time_launches(lambda: ll.lincomp(user, item, W, out=Y, bias=p["bias"], act="gelu"), steps, warmup, stream)

    def unfused():
        ll.lincomp(user, item, W, out=Y)
        torch.nn.functional.gelu(Y + p["b16"])

    _log(f"{c.name}: timing the layer + separate bias and GELU passes")
    tu = _time_launches(unfused, steps, warmup, stream)
    ev = tf["ms"]
    return dict(case=c, fused_ms=ev, median_ms=tf["median_ms"], unfused_ms=tu["ms"], req_s=c.R / (ev * 1e-3),
                gbs=c.algorithmic_bytes / (ev * 1e-3) / 1e9)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on this host's cores
# ---------------------------------------------------------------------------

def host_info() -> dict:
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        m = re.search(r"^Model name:\s*(.+)$", out, re.M)
        model = m.group(1).strip() if m else None
    except Exception:
        pass
    if model is None:
        try:
            m = re.search(r"^model name\s*:\s*(.+)$", open("/proc/cpuinfo").read(), re.M)
            model = m.group(1).strip() if m else platform.processor()
        except OSError:
            model = platform.processor()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    import oracle
    return dict(cpu_model=model, os_cpu_count=os.cpu_count(), usable_cpus=affinity,
                oracle_threads=oracle.get_threads())


def cpu_baseline_gemm(name: str, strip_rows: int | None = None):
    """The value-only oracle on the whole product (strip_rows None), or on a
    seeded strip of strip_rows rows plus the first and last rows, with the
    time for the whole shape extrapolated by row count and labelled so."""
    import numpy as np
    import oracle
    case = _case(name)
    if strip_rows is None:
        t0 = time.perf_counter()
        oracle.gemm_case(case, bound=False)
        dt = time.perf_counter() - t0
        return dict(workload=name, value=case.flops / dt / 1e12, unit="TFLOP/s", cores=oracle.get_threads(),
                    kind="oracle", seconds=round(dt, 3),
                    sample=f"fp64 oracle, whole C ({case.M}x{case.N}x{case.K})")
    start = int(np.random.default_rng(3).integers(0, case.M - strip_rows))
    rows_done, dt = 0, 0.0
    for r0, n in ((start, strip_rows), (0, 1), (case.M - 1, 1)):
        t0 = time.perf_counter()
        oracle.gemm_case(case, rows=(r0, n), bound=False)
        dt += time.perf_counter() - t0
        rows_done += n
    flops = 2.0 * rows_done * case.N * case.K
    return dict(workload=name, value=flops / dt / 1e12, unit="TFLOP/s", cores=oracle.get_threads(), kind="oracle",
                seconds=round(dt, 3), extrapolated_full_s=round(dt * case.M / rows_done, 1),
                sample=f"fp64 oracle, rows {start}..{start + strip_rows - 1}, 0 and {case.M - 1} of C "
                       f"({rows_done}x{case.N}x{case.K}); extrapolated_full_s scales the measured time by "
                       f"{case.M}/{rows_done} rows (extrapolated, not measured)")


def cpu_baseline_lincomp(name: str, target_s: float = 8.0):
    """The per-candidate (original, non-deduplicated) oracle on the first
    candidates of the workload, sized to about target_s of CPU time."""
    import oracle
    c = _case(name)
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
    return dict(workload=name, value=(n / c.C) / dt, unit="requests/s", cores=oracle.get_threads(),
                kind="oracle", seconds=round(dt, 3),
                sample=f"fp64 per-candidate oracle (each candidate's stacked input [user; item] "
                       f"materialised), first {n} of {c.R * c.C} candidates = {n / c.C:.1f} requests")


def vendor_context(steps: int, warmup: int):
    """torch.matmul on the GEMM workloads' shapes, operands of the same types
    and scales drawn on the device, timed like the library (same warm-up and
    step counts, per-call events)."""
    import torch
    import synth
    out = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    for name in ["gemm_4096", "ffn_up", "ffn_down", "gemm_3000", "gemm_4096_f16", "skinny_splitk", "gemm_4096_nt",
                 "gemm_4096_tn"]:
        M, N, K, kw = synth.GEMM_WORKLOADS[name]
        in_t = {"bf16": torch.bfloat16, "f16": torch.float16}[kw.get("in_dtype", "bf16")]

        def draw(rows, cols, dist):
            if dist[0] == "uniform":
                return (torch.rand(rows, cols, device="cuda", generator=gen) * (dist[2] - dist[1]) + dist[1]).to(in_t)
            return (torch.randn(rows, cols, device="cuda", generator=gen) * dist[2] + dist[1]).to(in_t)
        # column-major operands as transposed views (2-D products only)
        A = draw(K, M, kw["dist"]).t() if kw.get("a_col_major") else draw(M, K, kw["dist"])
        bd = kw.get("b_dist") or kw["dist"]
        B = draw(N, K, bd).t() if kw.get("b_col_major") else draw(K, N, bd)
        # torch.matmul writes C in its inputs' type: an fp32-output workload is
        # timed with a bf16/fp16 C (noted in the result)
        C = torch.empty(M, N, device="cuda", dtype=in_t)
        _log(f"vendor context: {name}")
        t = _time_launches(lambda: torch.matmul(A, B, out=C), steps, warmup, torch.cuda.current_stream())
        out.append(dict(workload=name, ms=round(t["ms"], 4), median_ms=round(t["median_ms"], 4),
                        tflops=round(2.0 * M * N * K / (t["ms"] * 1e-3) / 1e12, 1),
                        c_dtype=str(C.dtype).replace("torch.", ""), library_c_dtype=kw.get("out_dtype", "f32")))
        del A, B, C
        torch.cuda.empty_cache()
    return out


def _probe_lib():
    """libllprobes.so: the practical-ceiling probes (include/llprobes.h)."""
    import ctypes
    path = os.path.join(ROOT, "recsys_linear_layers_amd", "libllprobes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (run recsys_linear_layers_amd/build.py)")
    lib = ctypes.CDLL(path)
    lib.ll_probe_mfma_only.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ll_probe_mfma16_only.argtypes = lib.ll_probe_mfma_only.argtypes
    lib.ll_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.ll_probe_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_void_p]
    return lib


def _probe_call(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def mfma_probe(steps: int, warmup: int, grid: int = 1024, iters: int = 20000) -> dict:
    """bf16 MFMA issue with no memory traffic: grid workgroups of 4 waves, one
    per SIMD, each wave iters x 16 independent 32x32x16 MFMAs (or iters x 64
    of 16x16x32, twice the flops); once on small constant operands and once on
    random bf16 fragments (the multipliers switch as with a GEMM's data, and
    the chip's power limit sets the clock accordingly)."""
    import torch
    lib = _probe_lib()
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    frag = torch.randn(8 * 256 * 8, generator=gen, device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    res = {"probe": "mfma_only (bf16 MFMAs back to back, no memory traffic)", "grid": grid, "iters": iters}
    for shape, fn, flops in (("32x32x16", "ll_probe_mfma_only", grid * 4 * iters * 16 * 32768),
                             ("16x16x32", "ll_probe_mfma16_only", grid * 4 * iters * 64 * 16384)):
        call = getattr(lib, fn)
        sub = {"instruction": f"v_mfma_f32_{shape}_bf16", "flops_per_call": flops}
        for key, ptr in (("constant_operands", None), ("random_operands", frag.data_ptr())):
            _log(f"mfma probe {shape} ({key}): {grid} workgroups x {iters} iterations")
            t = _time_launches(lambda: _probe_call(call(grid, iters, ptr, out.data_ptr(), stream.cuda_stream), fn),
                               steps, warmup, stream)
            tf = flops / (t["ms"] * 1e-3) / 1e12
            sub[key] = {"ms": round(t["ms"], 4), "median_ms": round(t["median_ms"], 4), "TFLOP/s": round(tf, 1),
                        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        res[shape] = sub
    return res


def hbm_probe(mib: int, steps: int, warmup: int) -> dict:
    """Streaming through HBM with 16-byte accesses: a copy (1 read : 1 write),
    4 streams read per stream written, and reads alone (one 16-byte result
    written per thread), mib MiB per stream, with plain and with non-temporal
    loads and stores, at several grid sizes; the best of each pass is its
    ceiling."""
    import torch
    lib = _probe_lib()
    n16 = (mib << 20) // 16
    x = torch.ones(4 * n16 * 4, dtype=torch.int32, device="cuda")
    y = torch.empty(n16 * 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"probe": "hbm streaming (16-byte loads and stores, no reuse)", "mib_per_stream": mib}
    for streams, key in ((1, "copy"), (4, "read4_write1")):
        nbytes = (streams + 1) * n16 * 16
        for hints, hk in ((0, "plain"), (3, "nontemporal")):
            runs = []
            for grid in (1024, 4096, 16384):
                _log(f"hbm probe: {key}, {hk}, grid {grid}")
                t = _time_launches(lambda: _probe_call(lib.ll_probe_stream(streams, hints, x.data_ptr(), y.data_ptr(),
                                                                           n16, grid, stream.cuda_stream),
                                                       "ll_probe_stream"), steps, warmup, stream)
                runs.append(dict(grid=grid, ms=round(t["ms"], 4), median_ms=round(t["median_ms"], 4),
                                 gbs=round(nbytes / (t["ms"] * 1e-3) / 1e9, 1)))
            best = max(runs, key=lambda r: r["gbs"])
            res[f"{key}_{hk}"] = dict(bytes_per_call=nbytes, best_gbs=best["gbs"], best_grid=best["grid"],
                                      frac_of_peak=round(best["gbs"] / PEAK_HBM_GBS, 4), runs=runs)
    yr = torch.empty(16384 * 256 * 4, dtype=torch.int32, device="cuda")
    for hints, hk in ((0, "plain"), (1, "nontemporal")):
        runs = []
        for grid in (1024, 4096, 16384):
            _log(f"hbm probe: read_only, {hk}, grid {grid}")
            nbytes = 4 * n16 * 16 + grid * 256 * 16
            t = _time_launches(lambda: _probe_call(lib.ll_probe_read(hints, x.data_ptr(), yr.data_ptr(), 4 * n16, grid,
                                                                     stream.cuda_stream), "ll_probe_read"),
                               steps, warmup, stream)
            runs.append(dict(grid=grid, ms=round(t["ms"], 4), median_ms=round(t["median_ms"], 4),
                             gbs=round(nbytes / (t["ms"] * 1e-3) / 1e9, 1)))
        best = max(runs, key=lambda r: r["gbs"])
        res[f"read_only_{hk}"] = dict(bytes_per_call=4 * n16 * 16, best_gbs=best["gbs"], best_grid=best["grid"],
                                      frac_of_peak=round(best["gbs"] / PEAK_HBM_GBS, 4), runs=runs)
    return res


# Legs timed before the headline, in this order (the long FFN calls first);
# the configurations whose oracle is timed too are listed in CPU_LEGS.
ALSO_ORDER = ["ffn_up", "ffn_down", "ffn_up_bias_gelu", "lincomp_256x128", "lincomp_256x128_stacked",
              "lincomp_256x128_bias_gelu", "lincomp_ragged_256", "edge", "skinny_splitk", "gemm_256", "gemm_3000",
              "gemm_4096_f16", "gemm_4096_nt", "gemm_4096_tn", "gemm_4096"]
# workload -> strip rows (None: the whole problem)
CPU_LEGS = {"gemm_256": None, "ffn_up": 64, "ffn_down": 64, "edge": None, "skinny_splitk": None}


def prep_leg(name: str, preps: dict) -> dict:
    """Inputs and plans of one workload (reusing another workload's device
    operands where it is defined on them)."""
    if name in EPILOGUE_NAMES:
        base = EPILOGUE_NAMES[name]
        if base not in preps:
            preps[base] = prep_gemm(base)
        return prep_epilogue(preps[base])
    if name in STACKED_NAMES:
        base = STACKED_NAMES[name]
        if base not in preps:
            preps[base] = prep_lincomp(base)
        return prep_stacked(preps[base])
    if name in LC_EPILOGUE_NAMES:
        base = LC_EPILOGUE_NAMES[name]
        if base not in preps:
            preps[base] = prep_lincomp(base)
        return prep_lc_epilogue(preps[base])
    if name in RAGGED_NAMES:
        return prep_ragged(name)
    if name in LINCOMP_NAMES:
        return prep_lincomp(name)
    return prep_gemm(name, TILE_RULE_NAMES.get(name))


def time_leg(name: str, p: dict, steps: int, warmup: int) -> tuple[dict, dict]:
    """Time one non-headline workload; returns (its entry of "also", the raw result)."""
    if name in EPILOGUE_NAMES:
        x = time_epilogue(p, steps, warmup)
        return dict(workload=name, ms=round(x["fused_ms"], 4), median_ms=round(x["median_ms"], 4),
                    value=round(x["tflops"], 1), unit="TFLOP/s", mfma_frac=round(x["tflops"] / PEAK_BF16_TFLOPS, 4),
                    unfused_ms=round(x["unfused_ms"], 4), fused_speedup=round(x["unfused_ms"] / x["fused_ms"], 3),
                    plan=x["plan"]), x
    if name in LC_EPILOGUE_NAMES:
        x = time_lc_epilogue(p, steps, warmup)
        return dict(workload=name, ms=round(x["fused_ms"], 4), median_ms=round(x["median_ms"], 4),
                    value=round(x["req_s"], 1), unit="requests/s", hbm_gbs=round(x["gbs"], 1),
                    hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4), unfused_ms=round(x["unfused_ms"], 4),
                    fused_speedup=round(x["unfused_ms"] / x["fused_ms"], 3)), x
    if name in STACKED_NAMES:
        x = time_stacked(p, steps, warmup)
        return dict(workload=name, ms=round(x["kernel_ms"], 4), median_ms=round(x["median_ms"], 4),
                    value=round(x["req_s"], 1), unit="requests/s", hbm_gbs=round(x["gbs"], 1),
                    hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4), bytes=x["stacked_bytes"],
                    user_once_ms=round(x["dedup_ms"], 4), user_once_speedup=round(x["speedup"], 3)), x
    if name in RAGGED_NAMES:
        x = time_ragged(p, steps, warmup)
        c = x["case"]
        return dict(workload=name, ms=round(x["kernel_ms"], 4), median_ms=round(x["median_ms"], 4),
                    value=round(x["req_s"], 1), unit="requests/s", candidates=c.Ctot,
                    candidates_per_request=[int(c.lengths.min()), round(float(c.lengths.mean()), 1),
                                            int(c.lengths.max())],
                    hbm_gbs=round(x["gbs"], 1), hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4)), x
    if name in LINCOMP_NAMES:
        x = time_lincomp(p, steps, warmup)
        return dict(workload=name, ms=round(x["kernel_ms"], 4), median_ms=round(x["median_ms"], 4),
                    value=round(x["req_s"], 1), unit="requests/s", hbm_gbs=round(x["gbs"], 1),
                    hbm_frac=round(x["gbs"] / PEAK_HBM_GBS, 4)), x
    x = time_gemm(p, steps, warmup)
    c = x["case"]
    # compulsory bytes: A and B read once, C written once (the bound of the
    # skinny split-K shape, whose arithmetic intensity is under the ridge)
    cb = c.M * c.K * 2 + c.K * c.N * 2 + c.M * c.N * {"bf16": 2, "f16": 2, "f32": 4}[c.out_dtype]
    gbs = cb / (x["kernel_ms"] * 1e-3) / 1e9
    entry = dict(workload=name, ms=round(x["kernel_ms"], 4), median_ms=round(x["median_ms"], 4),
                 value=round(x["tflops"], 1), unit="TFLOP/s", mfma_frac=round(x["tflops"] / PEAK_BF16_TFLOPS, 4),
                 compulsory_bytes=cb, hbm_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                 plan=x["plan"])
    if name in TILE_RULE_NAMES:
        y = time_gemm(p, steps, warmup, TILE_RULE_NAMES[name])
        entry.update(without_rule_ms=round(y["kernel_ms"], 4),
                     tile_rule_speedup=round(y["kernel_ms"] / x["kernel_ms"], 3), plan_without_rule=y["plan"])
    return entry, x


def lincomp_object(x: dict, cpu: dict | None, name: str) -> dict:
    """The linear-compression half of the metric: requests/s with its HBM roofline."""
    c = x["case"]
    return dict(metric="linear-compression requests/s", value=round(x["req_s"], 1), unit="requests/s",
                workload=name, ms_per_call=round(x["kernel_ms"], 4), median_ms=round(x["median_ms"], 4),
                config=dict(requests=c.R, candidates_per_request=c.C, user_rows=c.Nu, item_rows=c.Ni, dim=c.D,
                            out_rows=c.Mo, y_dtype="bf16", algorithmic_bytes=c.algorithmic_bytes),
                roofline=dict(bound="hbm", achieved=x["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=x["gbs"] / PEAK_HBM_GBS, traffic=_traffic_from_profiles(name)),
                cpu_baseline=cpu)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gemm_4096",
                    choices=sorted(GEMM_NAMES | LINCOMP_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true", help="time only the headline workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, --steps times "
                         "(calibrates the HBM byte counters of a profiler run); prints its own line")
    ap.add_argument("--vendor-context", action="store_true",
                    help="time torch.matmul (the vendor GEMM) on the GEMM workloads' shapes instead, for context")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the MFMA-issue ceiling probe (bf16 MFMAs back to back, no memory traffic), "
                         "--steps times; prints its own line")
    ap.add_argument("--hbm-probe-mib", type=int, default=0,
                    help="only run the HBM streaming ceiling probes (a copy, and 4 streams read per stream "
                         "written, plain and non-temporal) over this many MiB per stream, --steps times per grid "
                         "size; prints its own line")
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
        t = _time_launches(lambda: dst.copy_(src), args.steps, args.warmup, stream)
        print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": round(t["ms"], 4),
                          "median_ms": round(t["median_ms"], 4), "GB/s": round(2 * n / (t["ms"] * 1e-3) / 1e9, 1)}))
        return

    if args.stream_probe_mib:
        # out[i] = x[0][i] + x[1][i] + x[2][i] + x[3][i]: 4 bytes read per byte
        # written, a plain streaming pass with no reuse.
        n = (args.stream_probe_mib << 20) // 4
        x = torch.ones((4, n), dtype=torch.float32, device="cuda")
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        t = _time_launches(lambda: torch.sum(x, dim=0, out=y), args.steps, args.warmup, stream)
        rd, wr = 16 * n, 4 * n
        print(json.dumps({"probe": "stream 4 reads : 1 write", "bytes_read": rd, "bytes_written": wr,
                          "ms": round(t["ms"], 4), "GB/s": round((rd + wr) / (t["ms"] * 1e-3) / 1e9, 1)}))
        return

    if args.mfma_probe:
        print(json.dumps(mfma_probe(args.steps, args.warmup)))
        return

    if args.hbm_probe_mib:
        print(json.dumps(hbm_probe(args.hbm_probe_mib, args.steps, args.warmup)))
        return

    if args.vendor_context:
        print(json.dumps({"probe": "vendor GEMM (torch.matmul), context only", "steps": args.steps,
                          "warmup": args.warmup, "results": vendor_context(args.steps, args.warmup)}))
        return

    head = args.workload
    cpu_on = not args.no_cpu_baseline
    names = [] if args.no_also else [n for n in ALSO_ORDER if n != head]

    # 1. Every workload's inputs into HBM and its plans made, before any timing.
    preps = {}
    for name in names + [head]:
        if name not in preps:
            preps[name] = prep_leg(name, preps)
    torch.cuda.synchronize()

    # 2. Every other configuration, back to back, then the headline.
    also, lc = [], None
    for name in names:
        entry, x = time_leg(name, preps[name], args.steps, args.warmup)
        also.append(entry)
        if name in LINCOMP_NAMES:
            lc = x
    rule_context = {}
    if head in LINCOMP_NAMES:
        r = time_lincomp(preps[head], args.steps, args.warmup)
        lc = r
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
        r = time_gemm(preps[head], args.steps, args.warmup)
        c = r["case"]
        metric, unit, value = "bf16 GEMM TFLOP/s", "TFLOP/s", r["tflops"]
        roof = dict(bound="mfma", achieved=r["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=r["tflops"] / PEAK_BF16_TFLOPS, traffic=_traffic_from_profiles(head))
        config = dict(workload=head, M=c.M, N=c.N, K=c.K, a_layout="row-major",
                      b_layout="column-major" if c.sbk == 1 else "row-major",
                      c_dtype=c.out_dtype, flops=c.flops)
        plan = r["plan"]
        if head in TILE_RULE_NAMES:
            y = time_gemm(preps[head], args.steps, args.warmup, TILE_RULE_NAMES[head])
            rule_context = dict(without_rule_ms=round(y["kernel_ms"], 4), without_rule_tflops=round(y["tflops"], 1),
                                tile_rule_speedup=round(y["kernel_ms"] / r["kernel_ms"], 3),
                                plan_without_rule=y["plan"])
    preps.clear()
    torch.cuda.empty_cache()
    for name in list(_CASES):
        if not (cpu_on and (name in CPU_LEGS or name in LINCOMP_NAMES or name == head)):
            _drop_case(name)

    # 3. CPU baselines, after all GPU timing.
    cpu, cpus, host, lc_cpu = None, [], None, None
    if cpu_on:
        _log("cpu baselines (oracle)")
        host = host_info()
        if head in LINCOMP_NAMES:
            cpu = lc_cpu = cpu_baseline_lincomp(head)
        else:
            cpu = cpu_baseline_gemm(head)
            if lc is not None:
                lc_cpu = cpu_baseline_lincomp(lc["case"].name)
        gpu_by_name = {a["workload"]: a for a in also}
        for name, strip in CPU_LEGS.items():
            if name == head or name not in gpu_by_name:
                continue
            b = cpu_baseline_gemm(name, strip)
            g = gpu_by_name[name]
            b["gpu_value"] = g["value"]
            b["gpu_over_cpu"] = round(g["value"] / b["value"], 1)
            cpus.append(b)
            _drop_case(name)
        cpu = dict(cpu, sample=cpu["sample"])
        cpu.pop("workload", None)

    out = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["wall_ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": config, "roofline": roof, "cpu_baseline": cpu,
        "kernel_ms": round(r["kernel_ms"], 4), "kernel_median_ms": round(r["median_ms"], 4),
        "kernel_per_call_mean_ms": round(r["per_call_mean_ms"], 4),
        "timed_after": [a["workload"] for a in also],
        "plan": plan, **rule_context,
    }
    if lc is not None and head not in LINCOMP_NAMES:
        out["lincomp"] = lincomp_object(lc, lc_cpu, lc["case"].name)
    out["also"] = also
    if cpu_on:
        out["cpu_baselines"] = cpus
        out["host"] = host
    out["kernel_source_hash"] = _kernel_source_hash()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
