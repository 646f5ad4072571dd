// Instantiations of the persistent GEMM for A K-contiguous, B N-contiguous.
#include "kernels.hpp"

#define LL_AK true
#define LL_BK false
#define LL_F16 false

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

hipError_t launch_gemm_kn(int kind, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (kind) {
    LL_GEMM_KINDS(LL_KIND_CASE)
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ll
