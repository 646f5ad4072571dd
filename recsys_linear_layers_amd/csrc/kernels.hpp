// Kernel configurations and launch entry points shared by the host code and
// the per-layout instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace ll {

// Tile configurations: X(name, BM, BN, KT, WM, WN, NPROD, NLW, STAGES, EPI).
// WM x WN computing waves each own a (BM/WM) x (BN/WN) block of the tile;
// NPROD > 0 adds that many loading waves; with NPROD == 0 the computing waves
// load too, the first NLW of them (all if NLW == 0).  KT is the k depth of one
// ring slot; STAGES the ring's slot count; EPI marks kinds with fused-epilogue
// instantiations.
#define LL_GEMM_KINDS(X)                                                                                   \
  X(KIND_SQ8_K64, 256, 256, 64, 2, 4, 0, 0, 2, 0)    /* 8 waves (2 per SIMD) 128x64 each */              \
  X(KIND_SQ8_K32, 256, 256, 32, 2, 4, 0, 0, 4, 0)    /* same, 4 x 32 KB slots */                         \
  X(KIND_WIDE8_PC, 256, 128, 64, 2, 4, 4, 0, 3, 0)   /* 8 computing 128x32 + 4 loading waves */          \
  X(KIND_WIDE_PC, 256, 128, 64, 2, 2, 4, 0, 3, 1)    /* 4 computing 128x64 + 4 loading waves */          \
  X(KIND_WIDE_COOP, 256, 128, 64, 2, 2, 0, 0, 3, 0)  /* 4 waves 128x64, load + compute */                \
  X(KIND_TALL_PC, 128, 256, 64, 2, 2, 4, 0, 3, 1)    /* skinny M: 4 computing 64x128 + 4 loading */      \
  X(KIND_SMALL_COOP, 128, 128, 64, 2, 2, 0, 0, 3, 0) /* small problems: 4 waves 64x64 */                 \
  X(KIND_T192_PC, 192, 256, 64, 2, 4, 4, 0, 2, 1)    /* 8 computing 96x64 + 4 loading; K-contiguous A */ \
  X(KIND_SQ8_LW4, 256, 256, 64, 4, 2, 0, 4, 2, 0)    /* 8 waves 64x128, one per SIMD also loads */

enum KernelKind {
#define LL_KIND_ENUM(name, ...) name,
  LL_GEMM_KINDS(LL_KIND_ENUM)
#undef LL_KIND_ENUM
  // 256x256 tile, four waves of 128x128 (one per SIMD), hand-ordered k-loop
  // (gemm_sq4.hpp); A K-contiguous, B N-contiguous, K a multiple of 64.
  KIND_SQ4_HO,
  KIND_COUNT
};

struct KindInfo {
  int bm, bn, kt, threads, lds, stages, nprod;
  int epi;  // has fused-epilogue instantiations
  const char* name;
};
const KindInfo& kind_info(int kind);

// Layout index: bit 1 = A is M-contiguous, bit 0 = B is N-contiguous.
inline int layout_index(bool a_kmajor, bool b_kmajor) { return (a_kmajor ? 0 : 2) | (b_kmajor ? 0 : 1); }

// Launch switch over every kind for one operand layout (instantiated once per layout).
#define LL_KIND_CASE(name, bm, bn, kt, wm, wn, np, lw, st, ep) \
  case name: return launch_cfg<GemmCfg<bm, bn, kt, wm, wn, np, st, LL_AK, LL_BK, LL_F16, 0, lw>>(a, grid, s);
#define LL_KIND_CASE_EPI(name, bm, bn, kt, wm, wn, np, lw, st, ep) \
  case name: return launch_epi<bm, bn, kt, wm, wn, np, lw, st, ep>(a, epi, grid, s);

// Launch `kind` for layout `layout` (bf16 or, f16 != 0, fp16 operands) on
// `grid` workgroups.  Returns the launch status.
hipError_t launch_gemm(int layout, int kind, int f16, const GemmKArgs& args, int grid, hipStream_t stream);
// The same with fused epilogue `epi` (1 + activation code: 1 bias only, 2
// ReLU, 3 GELU, 4 SiLU); only kinds marked in LL_GEMM_KINDS have these.
hipError_t launch_gemm_epi(int layout, int kind, int f16, int epi, const GemmKArgs& args, int grid,
                           hipStream_t stream);

// The hand-ordered 256x256 kind (gemm_sq4.hip): layout 1 (A K-contiguous,
// B N-contiguous) only; epi as for launch_gemm_epi (0: plain).
hipError_t launch_gemm_sq4(int layout, int f16, int epi, const GemmKArgs& args, int grid, hipStream_t stream);
hipError_t launch_gemm_sq4_bk(int f16, int epi, const GemmKArgs& args, int grid, hipStream_t stream);
hipError_t launch_gemm_sq4_am(int f16, int epi, const GemmKArgs& args, int grid, hipStream_t stream);
hipError_t launch_gemm_sq4_am_bk(int f16, int epi, const GemmKArgs& args, int grid, hipStream_t stream);

// Fused linear-compression kernel (lincomp_kernel.hpp).
struct LincompKArgs;
struct LincompKind {
  int bm, bn, kt, threads;
  const char* name;
};
const LincompKind& lincomp_kind();
// act: activation of the fused epilogue (0 none, 1 ReLU, 2 GELU, 3 SiLU); the
// bias, if any, is args.bias.
hipError_t launch_lincomp(const LincompKArgs& args, int act, int grid, hipStream_t stream);

// Auxiliary kernels.
hipError_t launch_pack_kmajor(const uint16_t* src, int64_t s_r, int64_t s_k, int64_t rows, int64_t K,
                              uint16_t* dst, int64_t ldp, hipStream_t stream);
hipError_t launch_pack_mnmajor(const uint16_t* src, int64_t s_r, int64_t s_k, int64_t rows, int64_t K,
                               uint16_t* dst, int64_t ldp, hipStream_t stream);
hipError_t launch_splitk_reduce(const float* partial, int splits, int64_t M, int64_t N, void* C,
                                int64_t ldcm, int64_t ldcn, int c_fmt, const float* bias, int act,
                                hipStream_t stream);
hipError_t launch_fill_zero(void* C, int64_t M, int64_t N, int64_t ldcm, int64_t ldcn, int c_fmt, const float* bias,
                            int act,
                            hipStream_t stream);
// Finishes the hand-ordered kind's K-split last-round tiles (tail_reduce_kernel).
hipError_t launch_tail_reduce(const float* partial, int splits, int tail_first, int tail_tiles, int tiles_m,
                              int tiles_n, int group_m, int64_t M, int64_t N, void* C, int64_t ldcm, int64_t ldcn,
                              int c_fmt, const float* bias, int act, hipStream_t stream);
// Zeroes n 32-bit words with one workgroup (a kernel, so that it may sit in a captured graph).
hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream);

}  // namespace ll
