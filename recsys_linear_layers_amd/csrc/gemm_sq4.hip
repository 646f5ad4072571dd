// Launch of the hand-ordered 256x256 GEMM kind (gemm_sq4.hpp), plain or with
// a fused epilogue; B N-contiguous.
#include "kernels.hpp"
#include "gemm_sq4.hpp"

namespace ll {

// layout 1: A K-contiguous, B N-contiguous (here); the other three layouts
// in units of their own (gemm_sq4_bk.hip, gemm_sq4_am.hip,
// gemm_sq4_am_bk.hip), so that the four build in parallel: 0 both
// K-contiguous, 2 A M-contiguous and B K-contiguous, 3 A M-contiguous and B
// N-contiguous
hipError_t launch_gemm_sq4(int layout, int f16, int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  if (layout == 1)
    return f16 ? launch_sq4<true, false, false>(epi, a, grid, s) : launch_sq4<false, false, false>(epi, a, grid, s);
  if (layout == 0) return launch_gemm_sq4_bk(f16, epi, a, grid, s);
  if (layout == 2) return launch_gemm_sq4_am_bk(f16, epi, a, grid, s);
  if (layout == 3) return launch_gemm_sq4_am(f16, epi, a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace ll
