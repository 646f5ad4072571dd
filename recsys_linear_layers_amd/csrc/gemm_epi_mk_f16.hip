// Instantiations of the persistent GEMM with a fused epilogue (bias and
// activation), fp16 operands, A M-contiguous, B K-contiguous.
#include "kernels.hpp"

#define LL_AK false
#define LL_BK true
#define LL_F16 true

namespace ll {

template <class Cfg>
static hipError_t launch_cfg(const GemmKArgs& a, int grid, hipStream_t s) {
  if constexpr (!Cfg::VALID) {
    return hipErrorInvalidValue;  // the plan never selects such a kind for this layout
  } else {
    hipLaunchKernelGGL(gemm_persistent<Cfg>, dim3(grid), dim3(Cfg::THREADS), 0, s, a);
    return hipGetLastError();
  }
}

template <int BM, int BN, int KT, int WM, int WN, int NP, int LW, int ST, int EP>
static hipError_t launch_epi(const GemmKArgs& a, int epi, int grid, hipStream_t s) {
  if constexpr (EP == 0) {
    return hipErrorInvalidValue;
  } else {
    switch (epi) {
      case 1: return launch_cfg<GemmCfg<BM, BN, KT, WM, WN, NP, ST, LL_AK, LL_BK, LL_F16, 1, LW>>(a, grid, s);
      case 2: return launch_cfg<GemmCfg<BM, BN, KT, WM, WN, NP, ST, LL_AK, LL_BK, LL_F16, 2, LW>>(a, grid, s);
      case 3: return launch_cfg<GemmCfg<BM, BN, KT, WM, WN, NP, ST, LL_AK, LL_BK, LL_F16, 3, LW>>(a, grid, s);
      case 4: return launch_cfg<GemmCfg<BM, BN, KT, WM, WN, NP, ST, LL_AK, LL_BK, LL_F16, 4, LW>>(a, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_gemm_epi_mk_f16(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    LL_GEMM_KINDS(LL_KIND_CASE_EPI)
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ll
