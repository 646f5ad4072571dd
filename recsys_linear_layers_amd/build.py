"""Compile the HIP sources under csrc/ for gfx950 into liblinlayers.so (in-tree),
and the measurement probes under probes/ into libllprobes.so.

Each .hip file is compiled to an object in parallel, then linked into its
shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblinlayers.so")
PROBES = os.path.join(HERE, "probes")
PROBE_LIB = os.path.join(HERE, "libllprobes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
# iterative-ilp: the machine scheduler then issues the next k-step's LDS fragment
# reads ahead of the current k-step's MFMAs instead of minimising registers.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr, flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)


# Units built with the compiler's default machine scheduler instead: the
# linear-compression kernels are bound by HBM, not by their instruction
# schedule, and iterative-ilp spilled their fused-epilogue instantiations
# (bias + GELU 34 registers against 10).
DEFAULT_SCHED = {"lincomp.hip"}


def _flags(src):
    if os.path.basename(src) not in DEFAULT_SCHED:
        return FLAGS
    out, i = [], 0
    while i < len(FLAGS):
        if FLAGS[i] == "-mllvm" and FLAGS[i + 1].startswith("-amdgpu-sched-strategy="):
            i += 2
            continue
        out.append(FLAGS[i])
        i += 1
    return out


# gemm_inst.hip is compiled once per operand layout (A K- or M-contiguous, B K-
# or N-contiguous), operand type (bf16, fp16) and epilogue (plain, fused), each
# unit defining the launch function that aux_kernels.hip dispatches to.
LAYOUTS = {"kk": (1, 1), "kn": (1, 0), "mk": (0, 1), "mn": (0, 0)}


def _units():
    """(source, object, extra flags) for every compile unit."""
    units = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        if os.path.basename(src) == "gemm_inst.hip":
            continue
        units.append((src, os.path.join(BUILD, os.path.basename(src)[:-4] + ".o"), []))
    inst = os.path.join(CSRC, "gemm_inst.hip")
    for epi in (0, 1):
        for lay, (ak, bk) in LAYOUTS.items():
            for f16 in (0, 1):
                name = "launch_gemm_" + ("epi_" if epi else "") + lay + ("_f16" if f16 else "")
                defs = [f"-DLL_AK={ak}", f"-DLL_BK={bk}", f"-DLL_F16={f16}", f"-DLL_EPI={epi}",
                        f"-DLL_LAUNCH={name}"]
                units.append((inst, os.path.join(BUILD, name + ".o"), defs))
    return units


def _probe_units():
    return [(src, os.path.join(BUILD, "probe_" + os.path.basename(src)[:-4] + ".o"), [])
            for src in sorted(glob.glob(os.path.join(PROBES, "*.hip")))]


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    units, probes = _units(), _probe_units()
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda u: _run([HIPCC, *_flags(u[0]), *u[2], "-c", u[0], "-o", u[1]], verbose), units + probes))
    # objects of sources that no longer exist are not linked
    _link([u[1] for u in units], LIB, verbose)
    _link([u[1] for u in probes], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
