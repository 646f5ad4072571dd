// Instantiations of the persistent GEMM for one operand layout and operand
// type, with or without fused epilogues.  build.py compiles this file once
// per combination, defining:
//   LL_AK      1: A K-contiguous, 0: A M-contiguous
//   LL_BK      1: B K-contiguous, 0: B N-contiguous
//   LL_F16     1: fp16 operands, 0: bf16
//   LL_EPI     1: the fused-epilogue instantiations (bias, activation), 0: plain
//   LL_LAUNCH  name of the launch function this unit defines
#include "kernels.hpp"

#if !defined(LL_AK) || !defined(LL_BK) || !defined(LL_F16) || !defined(LL_EPI) || !defined(LL_LAUNCH)
#error "gemm_inst.hip is compiled with -DLL_AK=.. -DLL_BK=.. -DLL_F16=.. -DLL_EPI=.. -DLL_LAUNCH=.."
#endif

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

#if LL_EPI
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

hipError_t LL_LAUNCH(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    LL_GEMM_KINDS(LL_KIND_CASE_EPI)
    default: return hipErrorInvalidValue;
  }
}
#else
hipError_t LL_LAUNCH(int kind, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    LL_GEMM_KINDS(LL_KIND_CASE)
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace ll
