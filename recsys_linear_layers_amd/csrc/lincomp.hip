// Instantiation and launch of the fused linear-compression kernel.
#include "kernels.hpp"
#include "lincomp_kernel.hpp"

namespace ll {

// 64 (Mo) x 256 (D) output tile, 64-deep slices, 4 computing waves (64 x 64
// each) + 4 loading waves, 3 ring slots (120 KB of LDS).
using LincompMain = LincompCfg<64, 256, 64, 4, 4, 3>;

const LincompKind& lincomp_kind() {
  static const LincompKind k = {LincompMain::BM, LincompMain::BN, LincompMain::KT, LincompMain::THREADS,
                                "lincomp_fused_64x256x64_s3_4c4p"};
  return k;
}

hipError_t launch_lincomp(const LincompKArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(lincomp_fused<LincompMain>, dim3(grid), dim3(LincompMain::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ll
