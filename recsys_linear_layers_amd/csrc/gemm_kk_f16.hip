// Instantiations of the persistent GEMM, fp16 operands, for A K-contiguous, B K-contiguous.
#include "kernels.hpp"

#define LL_AK true
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

hipError_t launch_gemm_kk_f16(int kind, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    LL_GEMM_KINDS(LL_KIND_CASE)
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ll
