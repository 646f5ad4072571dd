// Instantiations of the persistent GEMM for A K-contiguous,
// B N-contiguous.
#include "kernels.hpp"

namespace ll {

template <class Cfg>
static hipError_t launch_cfg(const GemmKArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_persistent<Cfg>, dim3(grid), dim3(Cfg::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_kn(int kind, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    case KIND_WIDE_PC: return launch_cfg<GemmCfg<256, 128, 2, 2, 4, 3, true, false>>(a, grid, s);
    case KIND_WIDE_COOP: return launch_cfg<GemmCfg<256, 128, 2, 2, 0, 3, true, false>>(a, grid, s);
    case KIND_TALL_PC: return launch_cfg<GemmCfg<128, 256, 2, 2, 4, 3, true, false>>(a, grid, s);
    case KIND_SMALL_COOP: return launch_cfg<GemmCfg<128, 128, 2, 2, 0, 3, true, false>>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ll
