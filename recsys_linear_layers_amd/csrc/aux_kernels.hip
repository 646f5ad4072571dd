// Auxiliary kernels: operand packing, split-K reduction, zero fill, and the
// launch table over the instantiation units of gemm_inst.hip (one per operand
// layout, operand type and epilogue).
#include "kernels.hpp"

namespace ll {

hipError_t launch_gemm_kk(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_kn(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_mk(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_mn(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_kk_f16(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_kn_f16(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_mk_f16(int kind, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_mn_f16(int kind, const GemmKArgs& a, int grid, hipStream_t s);

hipError_t launch_gemm(int layout, int kind, int f16, const GemmKArgs& args, int grid, hipStream_t stream) {
  if (kind == KIND_SQ4_HO) return launch_gemm_sq4(layout, f16, 0, args, grid, stream);
  if (f16) {
    switch (layout) {
      case 0: return launch_gemm_kk_f16(kind, args, grid, stream);
      case 1: return launch_gemm_kn_f16(kind, args, grid, stream);
      case 2: return launch_gemm_mk_f16(kind, args, grid, stream);
      case 3: return launch_gemm_mn_f16(kind, args, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (layout) {
    case 0: return launch_gemm_kk(kind, args, grid, stream);
    case 1: return launch_gemm_kn(kind, args, grid, stream);
    case 2: return launch_gemm_mk(kind, args, grid, stream);
    case 3: return launch_gemm_mn(kind, args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_epi_kk(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_kn(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_mk(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_mn(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_kk_f16(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_kn_f16(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_mk_f16(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);
hipError_t launch_gemm_epi_mn_f16(int kind, int epi, const GemmKArgs& a, int grid, hipStream_t s);

hipError_t launch_gemm_epi(int layout, int kind, int f16, int epi, const GemmKArgs& args, int grid,
                           hipStream_t stream) {
  if (kind == KIND_SQ4_HO) return launch_gemm_sq4(layout, f16, epi, args, grid, stream);
  switch (layout * 2 + (f16 ? 1 : 0)) {
    case 0: return launch_gemm_epi_kk(kind, epi, args, grid, stream);
    case 1: return launch_gemm_epi_kk_f16(kind, epi, args, grid, stream);
    case 2: return launch_gemm_epi_kn(kind, epi, args, grid, stream);
    case 3: return launch_gemm_epi_kn_f16(kind, epi, args, grid, stream);
    case 4: return launch_gemm_epi_mk(kind, epi, args, grid, stream);
    case 5: return launch_gemm_epi_mk_f16(kind, epi, args, grid, stream);
    case 6: return launch_gemm_epi_mn(kind, epi, args, grid, stream);
    case 7: return launch_gemm_epi_mn_f16(kind, epi, args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

const KindInfo& kind_info(int kind) {
#define LL_KIND_INFO(name, bm, bn, kt, wm, wn, np, lw, st, ep) \
  {bm, bn, kt, (wm * wn + np) * 64, st * (bm + bn) * kt * 2, st, np, ep, #name},
  static const KindInfo table[KIND_COUNT] = {LL_GEMM_KINDS(LL_KIND_INFO)
                                             {256, 256, 64, 256, 2 * 65536, 2, 0, 1, "KIND_SQ4_HO"}};
#undef LL_KIND_INFO
  return table[kind];
}

// dst[r][k] = src[r*s_r + k*s_k] for k < K, 0 for K <= k < ldp.  One thread per
// 8-element (16-byte) chunk of dst; rows along grid y.  When the source row
// is contiguous (s_k == 1) an interior chunk is read with aligned 32-bit
// loads: four words if its first element is 4-byte aligned, else the five
// words covering elements k0-1 .. k0+8, shifted by one element.  The first
// and last chunk of a row use element loads, so no load leaves the row.
__device__ __forceinline__ uint32_t pair16(uint32_t lo_word, uint32_t hi_word) {
  return (lo_word >> 16) | (hi_word << 16);  // elements 1 of lo_word and 0 of hi_word
}

__global__ void __launch_bounds__(256) pack_kmajor_kernel(const uint16_t* __restrict__ src, int64_t s_r,
                                                          int64_t s_k, int64_t rows, int64_t K,
                                                          uint16_t* __restrict__ dst, int64_t ldp) {
  const int64_t chunks_per_row = ldp / 8;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint16_t* row = src + r * s_r;
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < chunks_per_row;
         c += (int64_t)gridDim.x * blockDim.x) {
      const int64_t k0 = c * 8;
      uint4 o;
      if (s_k == 1 && k0 > 0 && k0 + 8 < K) {
        const uintptr_t a = (uintptr_t)(row + k0);
        if ((a & 3) == 0) {
          const uint32_t* w = (const uint32_t*)a;
          o.x = w[0];
          o.y = w[1];
          o.z = w[2];
          o.w = w[3];
        } else {
          const uint32_t* w = (const uint32_t*)(a - 2);  // elements k0-1, k0 | k0+1, k0+2 | ...
          const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
          o.x = pair16(w0, w1);
          o.y = pair16(w1, w2);
          o.z = pair16(w2, w3);
          o.w = pair16(w3, w4);
        }
      } else {
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (k0 + e < K) ? row[(k0 + e) * s_k] : (uint16_t)0;
        o.x = v[0] | ((uint32_t)v[1] << 16);
        o.y = v[2] | ((uint32_t)v[3] << 16);
        o.z = v[4] | ((uint32_t)v[5] << 16);
        o.w = v[6] | ((uint32_t)v[7] << 16);
      }
      *(uint4*)(dst + r * ldp + k0) = o;
    }
  }
}

hipError_t launch_pack_kmajor(const uint16_t* src, int64_t s_r, int64_t s_k, int64_t rows, int64_t K,
                              uint16_t* dst, int64_t ldp, hipStream_t stream) {
  const int64_t chunks = ldp / 8;
  if (rows == 0 || chunks == 0) return hipSuccess;
  const int64_t bx = (chunks + 255) / 256;
  const dim3 grid((unsigned)(bx < 64 ? bx : 64), (unsigned)(rows < 65535 ? rows : 65535));
  hipLaunchKernelGGL(pack_kmajor_kernel, grid, dim3(256), 0, stream, src, s_r, s_k, rows, K, dst, ldp);
  return hipGetLastError();
}

// dst[k][r] = src[r*s_r + k*s_k] for r < rows, 0 for rows <= r < ldp; k < K;
// ldp a multiple of 64 and dst 16-byte aligned.  The N-contiguous packed copy
// of B.  Each workgroup moves one 64 (k) x 64 (r) block through LDS: reads run
// along whichever source stride is 1 (a transpose when the source is
// K-contiguous, a copy when it is N-contiguous); a K-contiguous source row may
// start at any 2-byte offset, so its interior is read as aligned 32-bit words.
// Writes are 16-byte chunks along r.  Blocks along k are strided over grid y,
// so any K fits the grid.
__global__ void __launch_bounds__(256) pack_mnmajor_kernel(const uint16_t* __restrict__ src, int64_t s_r,
                                                           int64_t s_k, int64_t rows, int64_t K,
                                                           uint16_t* __restrict__ dst, int64_t ldp) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // [k][r]; 144-byte rows, 16-byte aligned
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const bool along_k = s_k == 1;
  const int t = threadIdx.x;
  for (int64_t k0 = (int64_t)blockIdx.y * 64; k0 < K; k0 += (int64_t)gridDim.y * 64) {
    if (along_k) {
      // thread: row rr = t / 4, elements kk0 .. kk0+15 with kk0 = 16 * (t % 4).  Away from
      // the row's first element and from K, nine aligned words cover them (shifted by one
      // element when they start at an odd element); elsewhere element by element.
      const int rr = t >> 2, kk0 = (t & 3) * 16;
      const int64_t r = r0 + rr, k = k0 + kk0;
      if (r < rows && k >= 1 && k + 18 <= K) {
        const int64_t o = r * s_r + k;
        const int sh = (int)(((uintptr_t)(src + o) >> 1) & 1);  // word-aligned start: o - sh
        const uint32_t* w = (const uint32_t*)(src + (o - sh));
        uint32_t v[9];
#pragma unroll
        for (int j = 0; j < 9; ++j) v[j] = w[j];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int i = j + sh;
          tile[kk0 + j][rr] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
        }
      } else {
#pragma unroll 4
        for (int j = 0; j < 16; ++j)
          tile[kk0 + j][rr] = (r < rows && k + j < K) ? src[r * s_r + k + j] : (uint16_t)0;
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const int e = i * 256 + t;
        const int rr = e & 63, kk = e >> 6;
        const int64_t r = r0 + rr, k = k0 + kk;
        tile[kk][rr] = (r < rows && k < K) ? src[r * s_r + k * s_k] : (uint16_t)0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * 256 + t;  // 16-byte chunk: k-row c / 8, elements 8 * (c % 8) ..
      const int kk = c >> 3, rr = (c & 7) * 8;
      const int64_t k = k0 + kk;
      if (k < K) *(uint4*)(dst + k * ldp + r0 + rr) = *(const uint4*)&tile[kk][rr];
    }
    __syncthreads();  // the tile is refilled for the next block along k
  }
}

hipError_t launch_pack_mnmajor(const uint16_t* src, int64_t s_r, int64_t s_k, int64_t rows, int64_t K,
                               uint16_t* dst, int64_t ldp, hipStream_t stream) {
  if (K == 0 || ldp == 0) return hipSuccess;
  if (ldp % 64 != 0 || ((uintptr_t)dst & 15)) return hipErrorInvalidValue;
  const int64_t bx = ldp / 64, by = (K + 63) / 64;
  if (bx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)bx, (unsigned)(by < 65535 ? by : 65535));
  hipLaunchKernelGGL(pack_mnmajor_kernel, grid, dim3(256), 0, stream, src, s_r, s_k, rows, K, dst, ldp);
  return hipGetLastError();
}

// C[i][j] = sum over s = 0..splits-1 (ascending) of partial[s][i][j].
// Bias and activation of the GEMM epilogue, selected at run time (these
// kernels are element-wise).
__device__ __forceinline__ float epi_rt(float z, float b, int act) {
  switch (act) {
    case 1: return epi<1>(z, b);
    case 2: return epi<2>(z, b);
    case 3: return epi<3>(z, b);
    default: return epi<0>(z, b);
  }
}

__device__ __forceinline__ void store_c(void* C, int64_t o, float v, int c_fmt) {
  if (c_fmt == 1)
    ((uint16_t*)C)[o] = f32_to_bf16_bits(v);
  else if (c_fmt == 2)
    ((uint16_t*)C)[o] = f32_to_f16_bits(v);
  else
    ((float*)C)[o] = v;
}

__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ P, int splits,
                                                            int64_t M, int64_t N, void* __restrict__ C,
                                                            int64_t ldcm, int64_t ldcn, int c_fmt,
                                                            const float* __restrict__ bias, int act) {
  const int64_t total = M * N;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    float acc = P[e];
    for (int s = 1; s < splits; ++s) acc += P[(int64_t)s * total + e];
    const int64_t i = e / N, j = e - i * N;
    store_c(C, i * ldcm + j * ldcn, epi_rt(acc, bias ? bias[j] : 0.f, act), c_fmt);
  }
}

// The same sums when N is a multiple of 4 (and the partials 16-byte aligned):
// rows along grid y, each thread four consecutive columns of a row with
// 16-byte loads, the splits added in the same ascending order per element
// (the same bits).  An fp32 C with unit column stride and a 16-byte aligned
// destination takes one 16-byte store.
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(const float* __restrict__ P, int splits, int64_t M,
                                                             int64_t N, void* __restrict__ C, int64_t ldcm,
                                                             int64_t ldcn, int c_fmt, const float* __restrict__ bias,
                                                             int act) {
  const int64_t total = M * N;
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (j >= N) return;
  for (int64_t i = blockIdx.y; i < M; i += gridDim.y) {
    const float* const q = P + i * N + j;
    f32x4 acc = *(const f32x4*)q;
    for (int s = 1; s < splits; ++s) acc += *(const f32x4*)(q + (int64_t)s * total);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = epi_rt(acc[e], bias ? bias[j + e] : 0.f, act);
    const int64_t o = i * ldcm + j * ldcn;
    if (c_fmt == 0 && ldcn == 1 && ((uintptr_t)((float*)C + o) & 15) == 0) {
      *(f32x4*)((float*)C + o) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_c(C, o + e * ldcn, v[e], c_fmt);
    }
  }
}

hipError_t launch_splitk_reduce(const float* partial, int splits, int64_t M, int64_t N, void* C,
                                int64_t ldcm, int64_t ldcn, int c_fmt, const float* bias, int act,
                                hipStream_t stream) {
  const int64_t total = M * N;
  if (total == 0) return hipSuccess;
  if (N % 4 == 0 && ((uintptr_t)partial & 15) == 0) {
    const int64_t bx = (N / 4 + 255) / 256;
    if (bx <= 0x7FFFFFFF) {
      const dim3 grid((unsigned)bx, (unsigned)(M < 65535 ? M : 65535));
      hipLaunchKernelGGL(splitk_reduce4_kernel, grid, dim3(256), 0, stream, partial, splits, M, N, C, ldcm, ldcn,
                         c_fmt, bias, act);
      return hipGetLastError();
    }
  }
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, stream, partial, splits, M, N, C,
                     ldcm, ldcn, c_fmt, bias, act);
  return hipGetLastError();
}

// The hand-ordered kind's last-round tiles that were split along K: tile
// tail_first + i (grouped order, 256x256) sums its splits' partials
// P[(i * splits + s)][256][256] in ascending s, then bias, activation and the
// C conversion.  Workgroup b takes rows 4 (b % 64) .. + 3 of tile b / 64,
// each thread four consecutive columns.
__global__ void __launch_bounds__(256) tail_reduce_kernel(const float* __restrict__ P, int splits, int tail_first,
                                                          int tiles_m, int tiles_n, int group_m, int64_t M,
                                                          int64_t N, void* __restrict__ C, int64_t ldcm,
                                                          int64_t ldcn, int c_fmt, const float* __restrict__ bias,
                                                          int act) {
  const int i = blockIdx.x >> 6;
  const int rl = 4 * (blockIdx.x & 63) + (threadIdx.x >> 6);
  const int cl = 4 * (threadIdx.x & 63);
  int tm, tn;
  grouped_tile(tail_first + i, tiles_m, tiles_n, group_m, tm, tn);
  const int64_t row = (int64_t)tm * 256 + rl;
  const int64_t col0 = (int64_t)tn * 256 + cl;
  if (row >= M || col0 >= N) return;
  const float* q = P + (int64_t)i * splits * 65536 + rl * 256 + cl;
  f32x4 acc = *(const f32x4*)q;
  for (int s = 1; s < splits; ++s) acc += *(const f32x4*)(q + (int64_t)s * 65536);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t col = col0 + e;
    if (col < N) store_c(C, row * ldcm + col * ldcn, epi_rt(acc[e], bias ? bias[col] : 0.f, act), c_fmt);
  }
}

hipError_t launch_tail_reduce(const float* partial, int splits, int tail_first, int tail_tiles, int tiles_m,
                              int tiles_n, int group_m, int64_t M, int64_t N, void* C, int64_t ldcm, int64_t ldcn,
                              int c_fmt, const float* bias, int act, hipStream_t stream) {
  if (tail_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(tail_reduce_kernel, dim3(tail_tiles * 64), dim3(256), 0, stream, partial, splits, tail_first,
                     tiles_m, tiles_n, group_m, M, N, C, ldcm, ldcn, c_fmt, bias, act);
  return hipGetLastError();
}

// K == 0: every sum is empty, so C = epilogue(0).
__global__ void __launch_bounds__(256) fill_zero_kernel(void* __restrict__ C, int64_t M, int64_t N,
                                                        int64_t ldcm, int64_t ldcn, int c_fmt,
                                                        const float* __restrict__ bias, int act) {
  const int64_t total = M * N;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / N, j = e - i * N;
    store_c(C, i * ldcm + j * ldcn, epi_rt(0.f, bias ? bias[j] : 0.f, act), c_fmt);
  }
}

__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* C, int64_t M, int64_t N, int64_t ldcm, int64_t ldcn, int c_fmt, const float* bias,
                            int act, hipStream_t stream) {
  const int64_t total = M * N;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, C, M, N, ldcm, ldcn, c_fmt, bias, act);
  return hipGetLastError();
}

}  // namespace ll
