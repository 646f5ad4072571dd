// Launch of the hand-ordered 256x256 GEMM kind (gemm_sq4.hpp), plain or with
// a fused epilogue.
#include "kernels.hpp"
#include "gemm_sq4.hpp"

namespace ll {

template <bool F16>
static hipError_t launch_sq4(int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_sq4<F16, 0>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 1: hipLaunchKernelGGL((gemm_sq4<F16, 1>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_sq4<F16, 2>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_sq4<F16, 3>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_sq4<F16, 4>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_sq4(int layout, int f16, int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  if (layout != 1) return hipErrorInvalidValue;  // A K-contiguous, B N-contiguous only
  return f16 ? launch_sq4<true>(epi, a, grid, s) : launch_sq4<false>(epi, a, grid, s);
}

}  // namespace ll
