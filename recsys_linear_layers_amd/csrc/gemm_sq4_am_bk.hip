// Launch of the hand-ordered 256x256 GEMM kind (gemm_sq4.hpp) with
// A M-contiguous and B K-contiguous, plain or with a fused epilogue.
#include "kernels.hpp"
#include "gemm_sq4.hpp"

namespace ll {

hipError_t launch_gemm_sq4_am_bk(int f16, int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  return f16 ? launch_sq4<true, true, true>(epi, a, grid, s) : launch_sq4<false, true, true>(epi, a, grid, s);
}

}  // namespace ll
