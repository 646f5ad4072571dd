"""Writes tests/golden/gemm_int_7x5x9.txt.  Calls only the oracle (and the
seeded input generator); the stored values never come from the HIP path."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
import synth  # noqa: E402

M, N, K = 7, 5, 9
A = synth.bf16_tensor(M * K, "int", -4, 4, seed=77, tensor=0)
B = synth.bf16_tensor(K * N, "int", -4, 4, seed=77, tensor=1)
C, _ = oracle.gemm(M, N, K, A, K, 1, B, N, 1)
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "gemm_int_7x5x9.txt"), "w") as f:
    f.write("# C = A.B (row-major A[M][K], B[K][N]); integer-valued bf16 inputs; values from the\n")
    f.write("# fp64 oracle (tests/golden/make_golden.py).  Lines: M N K / A / B / C\n")
    f.write(f"{M} {N} {K}\n")
    f.write(" ".join(str(int(v)) for v in synth.bf16_to_f32(A)) + "\n")
    f.write(" ".join(str(int(v)) for v in synth.bf16_to_f32(B)) + "\n")
    f.write(" ".join(repr(float(v)) for v in C.reshape(-1)) + "\n")
