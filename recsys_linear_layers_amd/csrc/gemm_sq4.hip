// Launch of the hand-ordered 256x256 GEMM kind (gemm_sq4.hpp).
#include "kernels.hpp"
#include "gemm_sq4.hpp"

namespace ll {

hipError_t launch_gemm_sq4(int layout, int f16, const GemmKArgs& a, int grid, hipStream_t s) {
  if (layout != 1) return hipErrorInvalidValue;  // A K-contiguous, B N-contiguous only
  if (f16)
    hipLaunchKernelGGL(gemm_sq4<true>, dim3(grid), dim3(Sq4::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_sq4<false>, dim3(grid), dim3(Sq4::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ll
