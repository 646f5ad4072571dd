// 256x256 GEMM kind with four waves of 128x128, one per SIMD, whose k-loop is
// a hand-ordered instruction stream (KIND_SQ4_HO).
//
// What is computed: C = A.B (fp32 accumulation) as in gemm_kernel.hpp, for A
// K-contiguous and B N-contiguous (row-major A and B, the layout the listings
// on "Triton 3.7 permite extender el compilador de GPU sin forks" state, and
// that of the FFN and square benchmark shapes), K a multiple of 64.
//
// Why a separate kind: a 128x128 wave tile reads a third less LDS per flop
// than the 64x128 tiles of the eight-wave kinds (256 rows x 64 k x 2 B of
// fragments per 2 x 128 x 128 x 64 flops), but it needs 256 fp32
// accumulators per lane, so it runs one wave per SIMD, and then no partner
// wave covers a wait: every fragment wait, load-issue stall and barrier wait
// idles the matrix unit.  The k-loop is therefore one inline-asm statement
// (gemm_sq4_loop.inc, written by gen_sq4_loop.py) that fixes the position of
// each wait, fragment read, direct-to-LDS load and barrier among the MFMAs;
// the accumulators live in a[0:255] for the whole work item.  Its MFMA is
// the 16x16x32 one (8 x 8 blocks per wave): for the same flops it moves half
// the accumulator bytes of the 32x32x16 one, and the power-limited clock is
// higher for it.
//
// Everything around the loop is ordinary code: per work item the tile's
// per-lane load offsets (lanes outside the matrix get an offset beyond the
// descriptor's num_records, so the hardware writes zeros), the first two
// slices' loads, and after the loop the epilogue, which reads the
// accumulators one 16x16 block at a time.
#pragma once

#include "gemm_kernel.hpp"
#include "gemm_sq4_loop.inc"

namespace ll {

struct Sq4 {
  static constexpr int BM = 256, BN = 256, KT = 64, THREADS = 256;
  static constexpr int SLOT = 65536, B_OFF = 32768, LDS = 2 * SLOT;
  // after the loop each wave stages its 128x128 block of a 16-bit C in an
  // image of 128 rows of 256 bytes plus 16 of padding, over the ring
  static constexpr int IMG_PITCH = 272, IMG = 128 * IMG_PITCH;
  // 256 bytes per wave above the ring and the images that the loop's L2
  // prefetches write into (nothing reads them; kept clear of the images so
  // that no prefetch still in flight can land in one)
  static constexpr int PF_OFF = 4 * IMG > LDS ? 4 * IMG : LDS;
  static constexpr int PF_LDS = LL_SQ4_PREFETCH ? 1024 : 0;
};

// Chunk swizzle of the A tile's rows (128 bytes, 8 chunks of 16 bytes each):
// chunk c of row r sits at c ^ sq4_swz_a(r).  A 16-byte fragment read gives
// lane l row l % 16 and chunk 4 kk + l / 16, and the LDS serves it in passes
// of lanes 8p..8p+7 with 32+8p..32+8p+7: 8 rows at chunks x and x ^ 2.  The
// four rows of each parity in such a pass then need one value from each of
// {0, 2}, {1, 3}, {4, 6}, {5, 7}, and eight consecutive rows eight distinct
// values: bits 0 and 1 of r swapped, and bit 1 flipped in the odd 8-row
// half.  Period 16 rows, so blocks 64 rows apart share addresses.
__device__ __forceinline__ int sq4_swz_a(int r) {
  return (((r & 1) << 1) | ((r >> 1) & 1) | (r & 4)) ^ (((r >> 3) & 1) << 1);
}

// Chunk swizzle of the B tile's k-rows (512 bytes, 32 chunks of 16 bytes
// each): chunk c of k-row kr sits at c ^ sq4_swz_b(kr).  A transposing B
// read serves 32 lanes at a time, and those take k-rows kr..kr+3 and
// kr+8..kr+11 at the same 16 columns; bits 0-1 of kr spread the first four
// over four bank groups and bit 3 moves the other four to four more, so the
// pass touches every bank once.  Bits 2 and 5 are left alone: the second
// half of a fragment (k-rows +4) and the next k32 step (k-rows +32) then sit
// at constant offsets from the first.
__device__ __forceinline__ int sq4_swz_b(int kr) { return ((kr & 3) << 2) | (((kr >> 3) & 1) << 1); }

// Longest wait at a round barrier, in ticks of the 100 MHz clock (30 us; the
// drift it corrects is a few us per round).
constexpr uint64_t kSyncWaitTicks = 3000;

// Accumulator block n (16x16; row block n / 8, column block n % 8 of the
// wave's 128x128): register r of lane l holds row 4 * (l / 16) + r, column
// l % 16 of the block (the output layout of v_mfma_f32_16x16x32).
#define LL_SQ4_ACC_FN(N)                                                                            \
  __device__ __forceinline__ f32x4 sq4_acc_##N() {                                                  \
    float r0, r1, r2, r3;                                                                          \
    asm volatile(LL_SQ4_READ_ACC_##N : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3));                    \
    return f32x4{r0, r1, r2, r3};                                                                  \
  }
LL_SQ4_BLOCKS(LL_SQ4_ACC_FN)
#undef LL_SQ4_ACC_FN

template <int N>
__device__ __forceinline__ f32x4 sq4_acc() {
#define LL_SQ4_ACC_PICK(n) \
  if constexpr (N == n) return sq4_acc_##n();
  LL_SQ4_BLOCKS(LL_SQ4_ACC_PICK)
#undef LL_SQ4_ACC_PICK
}

// The bias of the 8 columns this lane holds in the wave's 128 (one per column
// block), read once per tile; columns past N take none (they are not stored).
template <int EPI>
__device__ __forceinline__ void sq4_bias(const GemmKArgs& p, const TileInfo& ti, int wn0, int lane, float (&b)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = ti.n0 + wn0 + 16 * j + (lane & 15);
    b[j] = (EPI > 0 && col < p.N) ? bias_at(p, col) : 0.f;
  }
}

// Direct stores of block N: split-K partials (raw sums), or C of any type and
// layout with bias and activation, element by element with bounds checks
// (ragged tiles, fp32 C, C that the staged path does not take).
template <int EPI, int N>
__device__ __forceinline__ void sq4_store_block(const GemmKArgs& p, const TileInfo& ti, int wm0, int wn0, int lane,
                                                const float (&bias)[8]) {
  constexpr int I = N >> 3, J = N & 7;
  f32x4 v = sq4_acc<N>();
  const int col = ti.n0 + wn0 + 16 * J + (lane & 15);
  const int row0 = ti.m0 + wm0 + 16 * I + 4 * (lane >> 4);
  if (p.partial) {
    float* P = p.partial + (int64_t)ti.ks * p.M * p.N;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row0 + r < p.M && col < p.N) P[(int64_t)(row0 + r) * p.N + col] = v[r];
    return;
  }
  if constexpr (EPI > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = epi<EPI - 1>(v[r], bias[J]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + r;
    if (row < p.M && col < p.N) {
      const int64_t o = (int64_t)row * p.ldcm + (int64_t)col * p.ldcn;
      if (p.c_fmt == 1)
        ((uint16_t*)p.c)[o] = f32_to_bf16_bits(v[r]);
      else if (p.c_fmt == 2)
        ((uint16_t*)p.c)[o] = f32_to_f16_bits(v[r]);
      else
        ((float*)p.c)[o] = v[r];
    }
  }
}

// The round barrier's arrival: one lane of wave 0 adds 1 to its XCD's
// counter (a vector atomic) when cnt is set.
__device__ __forceinline__ void sq4_count_in(uint32_t* cnt, int wave, int lane) {
  if (cnt && wave == 0 && lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Work item t: a whole tile, or (from p.tail_first on) one K split of a tile
// of the last round, whose raw fp32 sums go to slot t - p.tail_first of
// p.tail_partial (slot -1 for a whole tile).
__device__ __forceinline__ TileInfo sq4_decode(const GemmKArgs& p, int t, int& slot) {
  if (t < p.tail_first) {
    slot = -1;
    return decode_tile<Sq4>(p, t);
  }
  slot = t - p.tail_first;
  TileInfo ti = decode_tile<Sq4>(p, p.tail_first + slot / p.tail_splits);
  ti.ks = slot % p.tail_splits;
  ti.kb = ti.ks * p.tail_kps;
  ti.ke = min(ti.kb + p.tail_kps, p.kiters);
  return ti;
}

// A K split's raw sums into its [256][256] fp32 partial tile (every element,
// also those past M or N: the reduce reads only those inside C).
template <int N>
__device__ __forceinline__ void sq4_tail_block(float* part, int wm0, int wn0, int lane) {
  constexpr int I = N >> 3, J = N & 7;
  const f32x4 v = sq4_acc<N>();
  float* q = part + (wm0 + 16 * I + 4 * (lane >> 4)) * 256 + wn0 + 16 * J + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) q[r * 256] = v[r];
}

__device__ __forceinline__ void sq4_tail_all(const GemmKArgs& p, int slot, int wm0, int wn0, int lane) {
  float* part = p.tail_partial + (int64_t)slot * (Sq4::BM * Sq4::BN);
#define LL_SQ4_TAIL(n) sq4_tail_block<n>(part, wm0, wn0, lane);
  LL_SQ4_BLOCKS(LL_SQ4_TAIL)
#undef LL_SQ4_TAIL
}

// Whole tiles of an fp32 C with unit column stride (any row stride): one
// base pointer per lane, the row offsets (16 I + r) * ldcm wave-uniform and
// the column block an immediate offset, so each element costs one store
// (the general path above spends ~10 operations per element on 64-bit
// offsets, bounds and the type).  Plain stores: with rows only 4-byte aligned
// a 64-byte row piece spans two cache lines, and L2 must merge the pieces of
// neighbouring column blocks (non-temporal stores were slower on every shape
// but one).
template <int EPI, int N>
__device__ __forceinline__ void sq4_store_f32_block(float* const (&rowp)[4], float bias) {
  f32x4 v = sq4_acc<N>();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = v[r];
    if constexpr (EPI > 0) x = epi<EPI - 1>(x, bias);
    rowp[r][16 * (N & 7)] = x;
  }
}

template <int EPI, int I>
__device__ __forceinline__ void sq4_store_f32_rows(const GemmKArgs& p, float* base, const float (&bias)[8]) {
  float* const rowp[4] = {base + (int64_t)(16 * I + 0) * p.ldcm, base + (int64_t)(16 * I + 1) * p.ldcm,
                          base + (int64_t)(16 * I + 2) * p.ldcm, base + (int64_t)(16 * I + 3) * p.ldcm};
  sq4_store_f32_block<EPI, 8 * I + 0>(rowp, bias[0]);
  sq4_store_f32_block<EPI, 8 * I + 1>(rowp, bias[1]);
  sq4_store_f32_block<EPI, 8 * I + 2>(rowp, bias[2]);
  sq4_store_f32_block<EPI, 8 * I + 3>(rowp, bias[3]);
  sq4_store_f32_block<EPI, 8 * I + 4>(rowp, bias[4]);
  sq4_store_f32_block<EPI, 8 * I + 5>(rowp, bias[5]);
  sq4_store_f32_block<EPI, 8 * I + 6>(rowp, bias[6]);
  sq4_store_f32_block<EPI, 8 * I + 7>(rowp, bias[7]);
}

template <int EPI>
__device__ __forceinline__ void sq4_store_f32_full(const GemmKArgs& p, const TileInfo& ti, int wm0, int wn0,
                                                   int lane) {
  float bias[8];
  sq4_bias<EPI>(p, ti, wn0, lane, bias);
  float* const base =
      (float*)p.c + (int64_t)(ti.m0 + wm0 + 4 * (lane >> 4)) * p.ldcm + ti.n0 + wn0 + (lane & 15);
  sq4_store_f32_rows<EPI, 0>(p, base, bias);
  sq4_store_f32_rows<EPI, 1>(p, base, bias);
  sq4_store_f32_rows<EPI, 2>(p, base, bias);
  sq4_store_f32_rows<EPI, 3>(p, base, bias);
  sq4_store_f32_rows<EPI, 4>(p, base, bias);
  sq4_store_f32_rows<EPI, 5>(p, base, bias);
  sq4_store_f32_rows<EPI, 6>(p, base, bias);
  sq4_store_f32_rows<EPI, 7>(p, base, bias);
}

template <int EPI>
__device__ __forceinline__ void sq4_store_all(const GemmKArgs& p, const TileInfo& ti, int wm0, int wn0, int lane) {
  float bias[8];
  sq4_bias<EPI>(p, ti, wn0, lane, bias);
#define LL_SQ4_STORE(n) sq4_store_block<EPI, n>(p, ti, wm0, wn0, lane, bias);
  LL_SQ4_BLOCKS(LL_SQ4_STORE)
#undef LL_SQ4_STORE
}

// Staged store of a wave's 128x128 block of 16-bit C through an LDS image
// (the ring is free once every wave has left the k-loop).  Per 16x16
// accumulator block each lane converts its column's four rows and writes
// them as four 16-bit values into the row-major [128][128] image.  Rows are
// 272 bytes apart, so row R starts 4 R banks further on: the four groups of
// 16 lanes of one write (rows 4 g + r) fall on banks 16 apart, and every
// address is one per-lane base plus an immediate.  That is eight vector ALU
// operations per block; with one wave per SIMD nothing hides their issue
// time, and exchanging values between lanes first, to write whole words,
// costs ten more.  Each 16-byte read then takes whole rows back and each
// lane stores 16 bytes, so a wave stores its block with 32 instructions of
// whole 128-byte lines instead of 256 of 2 bytes per lane.
__device__ __forceinline__ uint32_t sq4_stage_off(int row, int cb) { return (uint32_t)(row * Sq4::IMG_PITCH + cb); }

template <int EPI, int FMT, int N>
__device__ __forceinline__ void sq4_stage_block(int lane, const float (&bias)[8], char LL_LDS* img) {
  constexpr int I = N >> 3, J = N & 7;
  f32x4 v = sq4_acc<N>();
  if constexpr (EPI > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = epi<EPI - 1>(v[r], bias[J]);
  }
  // lane holds column 16 J + (lane & 15) of rows 16 I + 4 g + r, g = lane / 16
  const int row = 16 * I + 4 * (lane >> 4);
  const int cb = 32 * J + 2 * (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) *(uint16_t LL_LDS*)(img + sq4_stage_off(row + r, cb)) = to_c16<FMT>(v[r]);
}

template <int EPI, int FMT>
__device__ __forceinline__ void sq4_stage_all(const GemmKArgs& p, const TileInfo& ti, int wn0, int lane,
                                              char LL_LDS* img) {
  float bias[8];
  sq4_bias<EPI>(p, ti, wn0, lane, bias);
#define LL_SQ4_STAGE(n) sq4_stage_block<EPI, FMT, n>(lane, bias, img);
  LL_SQ4_BLOCKS(LL_SQ4_STAGE)
#undef LL_SQ4_STAGE
}

// The image back, four rows per read, each lane storing 16 bytes of a row:
// lanes 8p..8p+7 and 32+8p..32+8p+7, which one pass of a 16-byte LDS read
// serves together, take chunks 0-7 and 8-15 of row 4q+p (all 64 banks once),
// and each group of eight lanes stores a whole 128-byte line.  Element
// offsets fit in 32 bits (the fast-epilogue condition bounds ldcm * (M + 256)
// below 2^31), so each lane keeps one offset that steps by four rows.
__device__ __forceinline__ void sq4_flush(const GemmKArgs& p, const TileInfo& ti, int wm0, int wn0, int lane,
                                          const char LL_LDS* img) {
  const int pr = (lane >> 3) & 3, ch = ((lane >> 5) << 3) | (lane & 7);
  const int32_t step = 4 * (int32_t)p.ldcm;
  int32_t off = (ti.m0 + wm0 + pr) * (int32_t)p.ldcm + ti.n0 + wn0 + ch * 8;
  const char LL_LDS* const src = img + pr * Sq4::IMG_PITCH + ch * 16;
  uint16_t* const cb = (uint16_t*)p.c;
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const i32x4 v = *(const i32x4 LL_LDS*)(src + q * 4 * Sq4::IMG_PITCH);
    // C is not read again by this kernel: non-temporal (same box: +1.3% at
    // 4096^3, +1.5% at 8192^3, FFN shapes within noise)
    __builtin_nontemporal_store(v, (i32x4*)(cb + (uint32_t)off));
    off += step;
  }
}

// The first `count` of this wave's 16 direct-to-LDS loads of one slice into
// `slot`, in the loop's order (A 0, B 0, A 1, B 1, ..., or B first in each
// pair with LL_SQ4_B_FIRST).  Load q = wave + 4 i
// of an operand tile covers A rows 8q..8q+7 (K-contiguous, 128 bytes each) or
// B k-rows 2q, 2q+1 (512 bytes each) and lands at slot + q * 1024 (B tile at
// +32 KB).
template <int COUNT>
__device__ __forceinline__ void sq4_issue(i32x4 ra, i32x4 rb, const uint32_t (&va)[8], const uint32_t (&vb)[8],
                                          uint32_t ldsw, int slot, uint32_t soa, uint32_t sob) {
#pragma unroll
  for (int k = 0; k < COUNT; ++k) {
    const int i = k >> 1;
    if ((k & 1) != LL_SQ4_B_FIRST)
      dma16s(rb, ldsw + slot * Sq4::SLOT + Sq4::B_OFF + i * 4096, vb[i], sob);
    else
      dma16s(ra, ldsw + slot * Sq4::SLOT + i * 4096, va[i], soa);
  }
}

template <bool F16, int EPI, bool BK, bool AM>
__global__ void __launch_bounds__(Sq4::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
    gemm_sq4(const GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[Sq4::PF_OFF + Sq4::PF_LDS];
  char LL_LDS* smem = (char LL_LDS*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x;
  const int first = xcd_remap(blockIdx.x, gridDim.x);
  if (first >= p.total) return;  // uniform over the workgroup
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const uint32_t base = lds_u32(smem);

  // LDS addresses of this lane's fragment reads (16x16x32 operands: lane l
  // takes row / column l % 16 and k = 8 * (l / 16) .. + 7 of the step's 32).
  // A block i (16 rows) at k32 step kk: blocks i and i+4 share the swizzle
  // (rows 64 apart), so one address per (slot, kk, i % 4) serves both
  // (+8192).  B fragment j (16 columns): two transposing reads, each giving
  // a lane 4 k of its column; the swizzle (sq4_swz_b) ignores k-row bits 2
  // and 5, so step kk is +16384*kk and the second half (k-rows +4) +2048
  // from the step-0 address.  With B K-contiguous (BK) its tile is laid out
  // and read like A's: fbk, column blocks j and j+4 at +8192.  With A
  // M-contiguous (AM) its tile is laid out and read like an N-contiguous B's:
  // fat, row block i.
  uint32_t fa[2][2][4], fb[2][8], fbk[2][2][4], fat[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm0 + 16 * q + (lane & 15);
        const int lc = kk * 4 + (lane >> 4);
        fa[s][kk][q] = base + s * Sq4::SLOT + row * 128 + ((lc ^ sq4_swz_a(row)) << 4);
        const int col = wn0 + 16 * q + (lane & 15);
        fbk[s][kk][q] = base + s * Sq4::SLOT + Sq4::B_OFF + col * 128 + ((lc ^ sq4_swz_a(col)) << 4);
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = lane >> 4, sl = lane & 15;
      const int mn = wn0 + 16 * j + 4 * (sl & 3);
      const int kr = 8 * g + (sl >> 2);
      const int lc = mn >> 3, half = (mn & 7) * 2;
      fb[s][j] = base + s * Sq4::SLOT + Sq4::B_OFF + kr * 512 + ((lc ^ sq4_swz_b(kr)) << 4) + half;
      const int mr = wm0 + 16 * j + 4 * (sl & 3);
      fat[s][j] = base + s * Sq4::SLOT + kr * 512 + (((mr >> 3) ^ sq4_swz_b(kr)) << 4) + (mr & 7) * 2;
    }
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(base + wave * 1024);
  const uint32_t ldsp = __builtin_amdgcn_readfirstlane(base + Sq4::PF_OFF + wave * 256);
  const int lda = (int)p.a.ld, ldb = (int)p.b.ld;
  const uint32_t incb = BK ? 2u * Sq4::KT : 64u * 2u * (uint32_t)ldb;  // bytes of B per slice
  const uint32_t inca = AM ? 64u * 2u * (uint32_t)lda : 2u * Sq4::KT;  // and of A

  // Round barrier per XCD.  Work item t runs in round (t - first) / stride,
  // and the 32 workgroups of an XCD share panels only within a round.  Left
  // alone they drift apart by up to a whole tile over many rounds, and then
  // each fetches its panels' slices past L2 for itself.  So a workgroup
  // counts itself in once its work item is done (epilogue included: an
  // epilogue's length varies, and so would the next round's start) and,
  // before the next round's first loads, waits until every workgroup of its
  // XCD has done the same.  The wait is bounded (kSyncWaitTicks of the
  // 100 MHz clock), so a workgroup that is not resident costs time but never
  // blocks; the counts change no arithmetic.
  uint32_t* const cnt = p.sync ? p.sync + (blockIdx.x & 7) * 32 : nullptr;
  const uint32_t per_xcd = gridDim.x >> 3;
  uint32_t round = 0;
  for (int t = first; t < p.total; t += stride, ++round) {
    if (cnt && round > 0) {
      if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while ((uint32_t)__builtin_amdgcn_readfirstlane(
                   (int)__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < per_xcd * round) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncWaitTicks) break;
          __builtin_amdgcn_s_sleep(2);
        }
      }
      lds_barrier();
    }
    int slot;
    const TileInfo ti = sq4_decode(p, t, slot);
    int n = ti.ke - ti.kb;
    uint32_t va[8], vb[8], vpa = kOOB, vpb = kOOB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = wave + 4 * i;
      if constexpr (AM) {  // A k-rows 2q, 2q+1 like an N-contiguous B's
        const int kr = q * 2 + (lane >> 5);
        const int lca = (lane & 31) ^ sq4_swz_b(kr);
        va[i] = ti.m0 + lca * 8 < p.a.rows ? (uint32_t)(kr * lda + lca * 8) * 2u : kOOB;
      } else {
        const int row = q * 8 + (lane >> 3);
        const int lca = (lane & 7) ^ sq4_swz_a(row);
        va[i] = ti.m0 + row < p.a.rows ? (uint32_t)(row * lda + lca * 8) * 2u : kOOB;
      }
      if constexpr (BK) {  // B columns 8q.. like A rows
        const int col = q * 8 + (lane >> 3);
        const int lcb = (lane & 7) ^ sq4_swz_a(col);
        vb[i] = ti.n0 + col < p.b.rows ? (uint32_t)(col * ldb + lcb * 8) * 2u : kOOB;
      } else {
        const int kr = q * 2 + (lane >> 5);
        const int lcb = (lane & 31) ^ sq4_swz_b(kr);
        vb[i] = ti.n0 + lcb * 8 < p.b.rows ? (uint32_t)(kr * ldb + lcb * 8) * 2u : kOOB;
      }
    }
    // L2 prefetch offsets, one line per lane of this wave's share of a
    // slice: A rows 8q + t (q = wave + 4i) at their first chunk; B k-rows
    // 2q, 2q+1, four lines of 128 bytes each (a K-contiguous B: its rows 8q
    // + t, as A's).  kOOB: nothing is fetched.
    {
      const int q = wave + 4 * (lane >> 3);
      if constexpr ((LL_SQ4_PREFETCH & 2) != 0 && !AM) {
        const int row = q * 8 + (lane & 7);
        vpa = ti.m0 + row < p.a.rows ? (uint32_t)(row * lda) * 2u : kOOB;
      }
      if constexpr ((LL_SQ4_PREFETCH & 1) != 0) {
        if constexpr (BK) {
          const int col = q * 8 + (lane & 7);
          vpb = p.b_prefetch && ti.n0 + col < p.b.rows ? (uint32_t)(col * ldb) * 2u : kOOB;
        } else {
          const int kr = q * 2 + ((lane >> 2) & 1), line = lane & 3;
          vpb = p.b_prefetch && ti.n0 + line * 64 < p.b.rows ? (uint32_t)(kr * ldb + line * 64) * 2u : kOOB;
        }
      }
    }
    const int64_t oa = AM ? (int64_t)ti.kb * Sq4::KT * p.a.ld + ti.m0 : (int64_t)ti.m0 * p.a.ld + (int64_t)ti.kb * Sq4::KT;
    const int64_t ob = BK ? (int64_t)ti.n0 * p.b.ld + (int64_t)ti.kb * Sq4::KT
                          : (int64_t)ti.kb * Sq4::KT * p.b.ld + ti.n0;
    const i32x4 ra = make_rsrc(p.a.ptr + oa, clamp_records(p.a.extent - oa));
    const i32x4 rb = make_rsrc(p.b.ptr + ob, clamp_records(p.b.extent - ob));

    // slice 0, and of slice 1 the loads the loop would have issued after the
    // barrier of the slice before (all 16, or the first LL_SQ4_L3 when the
    // loop spreads the rest over the next slice's first steps)
    sq4_issue<16>(ra, rb, va, vb, ldsw, 0, 0u, 0u);
    if (n > 1) sq4_issue<LL_SQ4_L3>(ra, rb, va, vb, ldsw, 1, inca, incb);
    wait_vmcnt<0>();  // also covers the previous work item's stores
    lds_barrier();
    int m0v = 0;  // M0 is rewritten by the loop's loads

#define LL_SQ4_OPERANDS(FA, FB)                                                                               \
  : [n] "+s"(n), [m0] "+{m0}"(m0v)                                                                            \
  : [a0] "s"(ra[0]), [a1] "s"(ra[1]), [a2] "s"(ra[2]), [a3] "s"(ra[3]), [b0] "s"(rb[0]),                      \
    [b1] "s"(rb[1]), [b2] "s"(rb[2]), [b3] "s"(rb[3]), [incb] "s"(incb), [inca] "s"(inca), [ldsw] "s"(ldsw),  \
    [ldsp] "s"(ldsp),                                                                                         \
    [vpa] "v"(vpa), [vpb] "v"(vpb),                                                                           \
    [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [va4] "v"(va[4]),                 \
    [va5] "v"(va[5]), [va6] "v"(va[6]), [va7] "v"(va[7]), [vb0] "v"(vb[0]), [vb1] "v"(vb[1]),                 \
    [vb2] "v"(vb[2]), [vb3] "v"(vb[3]), [vb4] "v"(vb[4]), [vb5] "v"(vb[5]), [vb6] "v"(vb[6]),                 \
    [vb7] "v"(vb[7]), FA, FB                                                                                \
  : LL_SQ4_CLOBBERS
#define LL_SQ4_FA                                                                                             \
  [fa_0_0_0] "v"(fa[0][0][0]), [fa_0_0_1] "v"(fa[0][0][1]), [fa_0_0_2] "v"(fa[0][0][2]),                       \
      [fa_0_0_3] "v"(fa[0][0][3]), [fa_0_1_0] "v"(fa[0][1][0]), [fa_0_1_1] "v"(fa[0][1][1]),                   \
      [fa_0_1_2] "v"(fa[0][1][2]), [fa_0_1_3] "v"(fa[0][1][3]), [fa_1_0_0] "v"(fa[1][0][0]),                   \
      [fa_1_0_1] "v"(fa[1][0][1]), [fa_1_0_2] "v"(fa[1][0][2]), [fa_1_0_3] "v"(fa[1][0][3]),                   \
      [fa_1_1_0] "v"(fa[1][1][0]), [fa_1_1_1] "v"(fa[1][1][1]), [fa_1_1_2] "v"(fa[1][1][2]),                   \
      [fa_1_1_3] "v"(fa[1][1][3])
#define LL_SQ4_FAT                                                                                            \
  [fat_0_0] "v"(fat[0][0]), [fat_0_1] "v"(fat[0][1]), [fat_0_2] "v"(fat[0][2]), [fat_0_3] "v"(fat[0][3]),     \
      [fat_0_4] "v"(fat[0][4]), [fat_0_5] "v"(fat[0][5]), [fat_0_6] "v"(fat[0][6]), [fat_0_7] "v"(fat[0][7]), \
      [fat_1_0] "v"(fat[1][0]), [fat_1_1] "v"(fat[1][1]), [fat_1_2] "v"(fat[1][2]), [fat_1_3] "v"(fat[1][3]), \
      [fat_1_4] "v"(fat[1][4]), [fat_1_5] "v"(fat[1][5]), [fat_1_6] "v"(fat[1][6]), [fat_1_7] "v"(fat[1][7])
#define LL_SQ4_FB                                                                                             \
  [fb_0_0] "v"(fb[0][0]), [fb_0_1] "v"(fb[0][1]), [fb_0_2] "v"(fb[0][2]), [fb_0_3] "v"(fb[0][3]),             \
      [fb_0_4] "v"(fb[0][4]), [fb_0_5] "v"(fb[0][5]), [fb_0_6] "v"(fb[0][6]), [fb_0_7] "v"(fb[0][7]),         \
      [fb_1_0] "v"(fb[1][0]), [fb_1_1] "v"(fb[1][1]), [fb_1_2] "v"(fb[1][2]), [fb_1_3] "v"(fb[1][3]),         \
      [fb_1_4] "v"(fb[1][4]), [fb_1_5] "v"(fb[1][5]), [fb_1_6] "v"(fb[1][6]), [fb_1_7] "v"(fb[1][7])
#define LL_SQ4_FBK                                                                                            \
  [fbk_0_0_0] "v"(fbk[0][0][0]), [fbk_0_0_1] "v"(fbk[0][0][1]), [fbk_0_0_2] "v"(fbk[0][0][2]),                \
      [fbk_0_0_3] "v"(fbk[0][0][3]), [fbk_0_1_0] "v"(fbk[0][1][0]), [fbk_0_1_1] "v"(fbk[0][1][1]),            \
      [fbk_0_1_2] "v"(fbk[0][1][2]), [fbk_0_1_3] "v"(fbk[0][1][3]), [fbk_1_0_0] "v"(fbk[1][0][0]),            \
      [fbk_1_0_1] "v"(fbk[1][0][1]), [fbk_1_0_2] "v"(fbk[1][0][2]), [fbk_1_0_3] "v"(fbk[1][0][3]),            \
      [fbk_1_1_0] "v"(fbk[1][1][0]), [fbk_1_1_1] "v"(fbk[1][1][1]), [fbk_1_1_2] "v"(fbk[1][1][2]),            \
      [fbk_1_1_3] "v"(fbk[1][1][3])
    if constexpr (AM && BK) {
      if constexpr (F16)
        asm volatile(LL_SQ4_LOOP_F16_AM_BK LL_SQ4_OPERANDS(LL_SQ4_FAT, LL_SQ4_FBK));
      else
        asm volatile(LL_SQ4_LOOP_BF16_AM_BK LL_SQ4_OPERANDS(LL_SQ4_FAT, LL_SQ4_FBK));
    } else if constexpr (AM) {
      if constexpr (F16)
        asm volatile(LL_SQ4_LOOP_F16_AM LL_SQ4_OPERANDS(LL_SQ4_FAT, LL_SQ4_FB));
      else
        asm volatile(LL_SQ4_LOOP_BF16_AM LL_SQ4_OPERANDS(LL_SQ4_FAT, LL_SQ4_FB));
    } else if constexpr (BK) {
      if constexpr (F16)
        asm volatile(LL_SQ4_LOOP_F16_BK LL_SQ4_OPERANDS(LL_SQ4_FA, LL_SQ4_FBK));
      else
        asm volatile(LL_SQ4_LOOP_BF16_BK LL_SQ4_OPERANDS(LL_SQ4_FA, LL_SQ4_FBK));
    } else {
      if constexpr (F16)
        asm volatile(LL_SQ4_LOOP_F16 LL_SQ4_OPERANDS(LL_SQ4_FA, LL_SQ4_FB));
      else
        asm volatile(LL_SQ4_LOOP_BF16 LL_SQ4_OPERANDS(LL_SQ4_FA, LL_SQ4_FB));
    }
#undef LL_SQ4_FA
#undef LL_SQ4_FAT
#undef LL_SQ4_FB
#undef LL_SQ4_FBK
#undef LL_SQ4_OPERANDS

    lds_barrier();  // every wave is done reading the ring before it is reused
    if (slot >= 0) {  // a K split of a last-round tile: raw sums for the reduce
      sq4_tail_all(p, slot, wm0, wn0, lane);
      sq4_count_in(cnt, wave, lane);
      continue;
    }
    // a whole tile inside a 16-bit row-major C with 16-byte aligned rows:
    // staged through LDS (uniform over the workgroup)
    const bool staged = p.c_fast && p.c_fmt != 0 && ti.m0 + Sq4::BM <= p.M && ti.n0 + Sq4::BN <= p.N &&
                        ((uintptr_t)p.c & 15) == 0 && (p.ldcm & 7) == 0;
    if (staged) {
      char LL_LDS* img = smem + wave * Sq4::IMG;
      if (p.c_fmt == 1)
        sq4_stage_all<EPI, 1>(p, ti, wn0, lane, img);
      else
        sq4_stage_all<EPI, 2>(p, ti, wn0, lane, img);
      sq4_flush(p, ti, wm0, wn0, lane, img);
      sq4_count_in(cnt, wave, lane);
      // the next work item's loads land all over the LDS the other waves
      // may still be reading
      if (t + stride < p.total) lds_barrier();
      continue;
    }
    if (p.c_fmt == 0 && p.ldcn == 1 && !p.partial && ti.m0 + Sq4::BM <= p.M && ti.n0 + Sq4::BN <= p.N)
      sq4_store_f32_full<EPI>(p, ti, wm0, wn0, lane);
    else
      sq4_store_all<EPI>(p, ti, wm0, wn0, lane);
    sq4_count_in(cnt, wave, lane);
  }
}

// Launch of one instantiation by epilogue (0: none, 1: bias only, 2-4:
// ReLU, GELU, SiLU after the optional bias).
template <bool F16, bool BK, bool AM>
inline hipError_t launch_sq4(int epi, const GemmKArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case 0: hipLaunchKernelGGL((gemm_sq4<F16, 0, BK, AM>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 1: hipLaunchKernelGGL((gemm_sq4<F16, 1, BK, AM>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_sq4<F16, 2, BK, AM>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_sq4<F16, 3, BK, AM>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_sq4<F16, 4, BK, AM>), dim3(grid), dim3(Sq4::THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ll
