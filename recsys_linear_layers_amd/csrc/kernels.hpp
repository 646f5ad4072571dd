// Kernel configurations and launch entry points shared by the host code and
// the per-layout instantiation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace ll {

// Tile configurations (indices into the launch tables).
enum KernelKind {
  KIND_WIDE_PC = 0,   // 256x128 tile, 4 consumer waves (2x2, 128x64 each) + 4 producer waves, 3 stages
  KIND_WIDE_COOP,     // 256x128 tile, 4 waves that load and compute, 3 stages
  KIND_TALL_PC,       // 128x256 tile (skinny M), 4 consumers (2x2, 64x128) + 4 producers, 3 stages
  KIND_SMALL_COOP,    // 128x128 tile, 4 waves that load and compute (64x64 each), 3 stages
  KIND_LINCOMP_PC,    // 64x256 tile (one candidate's 64xD output), 4 consumers (1x4) + 4 producers
  KIND_COUNT
};

struct KindInfo {
  int bm, bn, threads, lds, stages, nprod;
  const char* name;
};
const KindInfo& kind_info(int kind);

// Layout index: bit 1 = A is M-contiguous, bit 0 = B is N-contiguous.
inline int layout_index(bool a_kmajor, bool b_kmajor) { return (a_kmajor ? 0 : 2) | (b_kmajor ? 0 : 1); }

// Launch `kind` for layout `layout` on `grid` workgroups.  Returns the launch status.
hipError_t launch_gemm(int layout, int kind, const GemmKArgs& args, int grid, hipStream_t stream);

// Auxiliary kernels.
hipError_t launch_pack_kmajor(const uint16_t* src, int64_t s_r, int64_t s_k, int64_t rows, int64_t K,
                              uint16_t* dst, int64_t ldp, hipStream_t stream);
hipError_t launch_splitk_reduce(const float* partial, int splits, int64_t M, int64_t N, void* C,
                                int64_t ldcm, int64_t ldcn, int c_bf16, hipStream_t stream);
hipError_t launch_fill_zero(void* C, int64_t M, int64_t N, int64_t ldcm, int64_t ldcn, int c_bf16,
                            hipStream_t stream);

}  // namespace ll
