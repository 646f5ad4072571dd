// Instantiation and launch of the fused linear-compression kernel.
#include <stdlib.h>

#include "kernels.hpp"
#include "lincomp_kernel.hpp"

namespace ll {

// Default: 64 (Mo) x 256 (D) output tile, 64-deep slices, 4 computing waves
// (64 x 64 each) + 4 loading waves, 3 ring slots (120 KB of LDS).
// Configurations X(BM, BN, KT, computing waves, loading waves, ring slots); the
// first is the default, LL_LINCOMP_CFG=<index> selects another (sweeps).
#define LL_LINCOMP_CFGS(X) \
  X(64, 256, 64, 4, 4, 3)  \
  X(64, 256, 64, 4, 4, 4)  \
  X(64, 256, 32, 4, 4, 4)  \
  X(64, 256, 32, 4, 4, 6)  \
  X(64, 256, 64, 4, 2, 3)  \
  X(64, 256, 32, 4, 2, 7)

static int cfg_index() {
  static const int idx = [] {
    const char* e = getenv("LL_LINCOMP_CFG");
    return e ? atoi(e) : 0;
  }();
  return idx;
}

const LincompKind& lincomp_kind() {
#define LL_LC_KIND(bm, bn, kt, nc, np, st) {bm, bn, kt, (nc + np) * 64, "lincomp_" #bm "x" #bn "x" #kt "_s" #st "_" #nc "c" #np "p"},
  static const LincompKind kinds[] = {LL_LINCOMP_CFGS(LL_LC_KIND)};
#undef LL_LC_KIND
  const int n = (int)(sizeof kinds / sizeof kinds[0]);
  const int i = cfg_index();
  return kinds[i >= 0 && i < n ? i : 0];
}

hipError_t launch_lincomp(const LincompKArgs& a, int act, int grid, hipStream_t s) {
  // A fused epilogue runs in the default configuration (one instantiation per
  // activation, with and without a bias); the sweep configurations are plain.
  if (act != 0 || a.bias || cfg_index() == 0) {
    const int v = act * 2 + (a.bias ? 1 : 0);
    switch (v) {
#define LL_LC_EPI(n, b)                                                                       \
  case n * 2 + b: {                                                                           \
    using C = LincompCfg<64, 256, 64, 4, 4, 3, n, b>;                                         \
    hipLaunchKernelGGL(lincomp_fused<C>, dim3(grid), dim3(C::THREADS), 0, s, a);              \
    return hipGetLastError();                                                                 \
  }
      LL_LC_EPI(0, 0)
      LL_LC_EPI(0, 1)
      LL_LC_EPI(1, 0)
      LL_LC_EPI(1, 1)
      LL_LC_EPI(2, 0)
      LL_LC_EPI(2, 1)
      LL_LC_EPI(3, 0)
      LL_LC_EPI(3, 1)
#undef LL_LC_EPI
      default: return hipErrorInvalidValue;
    }
  }
  int i = 0;
#define LL_LC_LAUNCH(bm, bn, kt, nc, np, st)                                                        \
  if (cfg_index() == i++) {                                                                        \
    using C = LincompCfg<bm, bn, kt, nc, np, st>;                                                  \
    hipLaunchKernelGGL(lincomp_fused<C>, dim3(grid), dim3(C::THREADS), 0, s, a);                   \
    return hipGetLastError();                                                                      \
  }
  LL_LINCOMP_CFGS(LL_LC_LAUNCH)
#undef LL_LC_LAUNCH
  using C = LincompCfg<64, 256, 64, 4, 4, 3>;
  hipLaunchKernelGGL(lincomp_fused<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ll
