// Practical-ceiling probes (include/llprobes.h): MFMA issue with no memory
// traffic, and plain HBM streaming with 16-byte accesses.  Measurement only:
// nothing here computes a library operation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/llprobes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 independent accumulators per wave (the 128x128 block of four 32x32
// tiles by four that a GEMM wave holds): an MFMA's result is next needed 16
// MFMAs later, far past its latency, so issue never waits on a dependency.
// Accumulator (i, j) takes A fragment i and B fragment j, as in a GEMM's
// k16 step.  Operands either come from `frag` (eight 16-byte fragments per
// lane, e.g. random bf16 patterns: the multipliers switch as with real data)
// or, with frag null, are small constants that barely switch (the issue
// rate with the least power).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_only_kernel(int iters, const uint4* __restrict__ frag, float* out) {
  bf16x8 a[4], b[4];
  if (frag) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __builtin_bit_cast(bf16x8, frag[i * 256 + threadIdx.x]);
      b[i] = __builtin_bit_cast(bf16x8, frag[(4 + i) * 256 + threadIdx.x]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[i][e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[i][e] = (__bf16)(float)((3 * threadIdx.x + e) & 7);
      }
  }
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j >> 2], b[j & 3], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The same with the 16x16x32 MFMA (the library's hand-ordered GEMM loop's):
// the 128x128 block as 8 x 8 accumulators of 16x16, 64 independent MFMAs per
// iteration (16384 flops each, twice the 32x32 probe's flops per
// iteration), A fragment i and B fragment j for accumulator (i, j).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma16_only_kernel(int iters, const uint4* __restrict__ frag, float* out) {
  bf16x8 a[8], b[8];
  if (frag) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = __builtin_bit_cast(bf16x8, frag[(i & 3) * 256 + threadIdx.x]);
      b[i] = __builtin_bit_cast(bf16x8, frag[(4 + (i & 3)) * 256 + ((threadIdx.x + 32 * (i >> 2)) & 255)]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[i][e] = (__bf16)(float)((threadIdx.x + e + i) & 7);
        b[i][e] = (__bf16)(float)((3 * threadIdx.x + e + i) & 7);
      }
  }
  f32x4 acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = f32x4{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 64; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j >> 3], b[j & 7], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride over n16 elements, U elements per thread per pass with all of
// a pass's loads issued before its stores; NT: bit 0 non-temporal loads, bit 1
// non-temporal stores.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int S, int NT>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                     int64_t n16) {
  constexpr int U = 4;
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += step) {
    u32x4 v[U][S];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (i < n16) {
          if constexpr (NT & 1)
            v[u][s] = __builtin_nontemporal_load(x + s * n16 + i);
          else
            v[u][s] = x[s * n16 + i];
        } else {
          v[u][s] = u32x4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) {
        u32x4 r = v[u][0];
#pragma unroll
        for (int s = 1; s < S; ++s) r ^= v[u][s];
        if constexpr (NT & 2)
          __builtin_nontemporal_store(r, y + i);
        else
          y[i] = r;
      }
    }
  }
}

// Read-only streaming: each thread XORs together every 16-byte element it
// reads and writes the one result at the end (16 bytes per thread, so the
// traffic is reads to within grid * 4 KiB).
template <int NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ x, u32x4* __restrict__ y, int64_t n16) {
  constexpr int U = 8;
  const int64_t step = (int64_t)gridDim.x * 256 * U;
  u32x4 r = u32x4{0, 0, 0, 0};
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) {
        if constexpr (NT)
          v[u] = __builtin_nontemporal_load(x + i);
        else
          v[u] = x[i];
      } else {
        v[u] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) r ^= v[u];
  }
  y[(int64_t)blockIdx.x * 256 + threadIdx.x] = r;
}

template <int S>
hipError_t launch_stream(int hints, const u32x4* x, u32x4* y, int64_t n16, int grid, hipStream_t st) {
  switch (hints) {
    case 0: stream_kernel<S, 0><<<grid, 256, 0, st>>>(x, y, n16); break;
    case 1: stream_kernel<S, 1><<<grid, 256, 0, st>>>(x, y, n16); break;
    case 2: stream_kernel<S, 2><<<grid, 256, 0, st>>>(x, y, n16); break;
    default: stream_kernel<S, 3><<<grid, 256, 0, st>>>(x, y, n16); break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" int ll_probe_mfma_only(int grid, int iters, const void* operands, float* out, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 0 || iters > (1 << 24) || !out) return -1;
  if ((uintptr_t)operands & 15) return -1;
  mfma_only_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(iters, (const uint4*)operands, out);
  return (int)hipGetLastError();
}

extern "C" int ll_probe_mfma16_only(int grid, int iters, const void* operands, float* out, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 0 || iters > (1 << 24) || !out) return -1;
  if ((uintptr_t)operands & 15) return -1;
  mfma16_only_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(iters, (const uint4*)operands, out);
  return (int)hipGetLastError();
}

extern "C" int ll_probe_stream(int streams, int hints, const void* x, void* y, int64_t n16, int grid, void* stream) {
  if ((streams != 1 && streams != 4) || hints < 0 || hints > 3 || n16 < 0 || grid < 1 || grid > (1 << 20))
    return -1;
  if (n16 == 0) return 0;
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return -1;
  const uintptr_t xb = (uintptr_t)x, xe = xb + (uintptr_t)(streams * n16 * 16);
  const uintptr_t yb = (uintptr_t)y, ye = yb + (uintptr_t)(n16 * 16);
  if (xb < ye && yb < xe) return -1;
  const u32x4* xp = (const u32x4*)x;
  u32x4* yp = (u32x4*)y;
  const hipError_t e = streams == 1 ? launch_stream<1>(hints, xp, yp, n16, grid, (hipStream_t)stream)
                                    : launch_stream<4>(hints, xp, yp, n16, grid, (hipStream_t)stream);
  return (int)e;
}

extern "C" int ll_probe_read(int hints, const void* x, void* y, int64_t n16, int grid, void* stream) {
  if (hints < 0 || hints > 1 || n16 < 0 || grid < 1 || grid > (1 << 20)) return -1;
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return -1;
  const uintptr_t xb = (uintptr_t)x, xe = xb + (uintptr_t)(n16 * 16);
  const uintptr_t yb = (uintptr_t)y, ye = yb + (uintptr_t)grid * 256 * 16;
  if (xb < ye && yb < xe) return -1;
  if (hints)
    read_kernel<1><<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)x, (u32x4*)y, n16);
  else
    read_kernel<0><<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)x, (u32x4*)y, n16);
  return (int)hipGetLastError();
}
