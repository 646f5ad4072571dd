// Persistent, software-pipelined bf16 GEMM for gfx950 (MI355X).
//
// What is computed: C = A.B (fp32 accumulation) over strided operands, as the
// listings on "Triton 3.7 permite extender el compilador de GPU sin forks"
// state the problem (sections "NVIDIA H100 (Hopper): GEMM persistente" and
// "AMD MI350: GEMM segmentado"), optionally batched, split along K, and with a
// per-batch fp32 bias added in the epilogue (used by the linear-compression
// layer).
//
// How (gfx950-specific design; the pages' TMA/WGMMA and register-staged
// mechanisms are not used):
//  * A ring of STAGES LDS slots.  Each slot holds one BK=64 k-slice of the A
//    tile and of the B tile.  Producer waves fill slots straight from HBM with
//    `buffer_load_dwordx4 ... lds` (no VGPR staging): each instruction moves
//    64 lanes x 16 B = 1 KB into a contiguous LDS block.  Out-of-range lanes get
//    an offset beyond the buffer's num_records, so the hardware writes zeros.
//  * Consumer waves read MFMA operand fragments from the slot computed STAGES-1
//    steps earlier and run v_mfma_f32_32x32x16_bf16.  A K-contiguous operand
//    is stored as [rows][64] (128-byte rows, 16-byte chunks XOR-swizzled) and
//    read with ds_read_b128; an M/N-contiguous operand is stored as it sits in
//    memory, [64][rows], and read with ds_read_b64_tr_b16, which transposes
//    16-bit elements across each group of 16 lanes.
//  * Handoff: one workgroup barrier per k-step.  Before it, producers wait
//    (vmcnt) until their loads for the slot about to be consumed have landed;
//    after it, producers refill the slot consumed in the previous step.  With
//    NPROD > 0 the roles are separate waves; with NPROD == 0 every wave does
//    both.  The ring runs across tile boundaries of the persistent loop.
//  * Persistent grid over (batch, k-split, tile) work items in grouped
//    (GROUP_M) order, with workgroup ids remapped so that the consecutive
//    work items that share operand panels land on the same XCD (and its L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LL_LDS __attribute__((address_space(3)))

constexpr int kBK = 64;                    // k elements per pipeline stage
constexpr uint32_t kOOB = 0x80000000u;     // byte offset beyond every num_records used here
constexpr uint32_t kRsrcWord3 = 0x00020000u;

struct OperandArgs {
  const uint16_t* ptr;  // element (0, 0) of batch 0
  int64_t ld;           // K-major: elements between MN rows; MN-major: elements between k rows
  int32_t rows;         // extent along M (A) or N (B)
  int32_t kvalid;       // k extent holding data; K-major operands: a multiple of 8
  int64_t bo, bi;       // batch offset of item b: (b / bdiv) * bo + (b % bdiv) * bi
  int64_t extent;       // elements addressable from ptr (clamps num_records)
};

struct GemmKArgs {
  OperandArgs a, b;
  void* c;
  int64_t ldcm, ldcn, cbo, cbi;
  const float* bias;  // optional fp32 addend, same batch/row/col indexing scheme as C
  int64_t bias_m, bias_n, bias_bo, bias_bi;
  float* partial;     // split-K partials [splits][M][N], or null
  int32_t M, N;
  int32_t c_bf16;
  int32_t bdiv;
  int32_t batches, splits, kiters, kps;
  int32_t tiles_m, tiles_n, group_m;
  int32_t total;
};

template <int BM_, int BN_, int WM_, int WN_, int NPROD_, int STAGES_, bool AK_, bool BK_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = WM_, WN = WN_;   // consumer-wave grid
  static constexpr int NCONS = WM * WN;
  static constexpr int NPROD = NPROD_;        // 0: every wave loads and computes
  static constexpr int STAGES = STAGES_;
  static constexpr bool A_KMAJOR = AK_;       // A stored K-contiguous (row-major A)
  static constexpr bool B_KMAJOR = BK_;       // B stored K-contiguous (column-major B)
  static constexpr int WAVES = NCONS + NPROD;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // 32x32 blocks per wave
  static constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2;
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGES * SLOT;
  static constexpr int LOADERS = NPROD ? NPROD : NCONS;
  static constexpr int QA = BM / 8, QB = BN / 8;           // 1-KB load instructions per stage
  static constexpr int LPW = (QA + QB) / LOADERS;           // per loading wave
  static_assert(QA % LOADERS == 0 && QB % LOADERS == 0, "load split");
  static_assert(FM >= 1 && FN >= 1 && BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(STAGES >= 2, "stages");
  static constexpr int WAVES_PER_EU = (WAVES + 3) / 4;
};

// ---------------------------------------------------------------------------
// LDS layouts.  K-major tile: [rows][64] bf16, 128-byte rows of eight 16-byte
// chunks; chunk c of row r sits at c ^ swz_k(r), which makes the 8 (or 16)
// rows one ds_read_b128 pass touches hit distinct banks.  MN-major tile:
// [64][rows] bf16; chunk c of k-row r sits at c ^ swz_mn(r), which spreads the
// 4 k-rows one ds_read_b64_tr_b16 lane group reads over different banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_k(int row) { return (row ^ (row >> 3)) & 7; }
template <int CH>
__device__ __forceinline__ int swz_mn(int k) { return ((k & 3) << 2) & (CH - 1); }

__device__ __forceinline__ uint32_t clamp_records(int64_t elems) {
  if (elems <= 0) return 0u;
  const int64_t bytes = elems * 2;
  return bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: 48-bit base, stride 0, num_records bytes; word 3 is
// the gfx9 raw-buffer format.  All fields wave-uniform (SGPRs).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nrec) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nrec);
  r[3] = (int)kRsrcWord3;
  return r;
}

// One direct-to-LDS load: lane l's 16 bytes at rsrc.base + voff land at LDS
// byte lds_addr + 16*l.  Written as inline asm so that the compiler does not
// treat every later LDS access as dependent on it (it would otherwise insert
// s_waitcnt vmcnt(0) before each ds_read and barrier).  Completion is tracked
// by the explicit vmcnt waits of the pipeline instead.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const char LL_LDS* p) { return (uint32_t)(uintptr_t)p; }

// Issue this wave's share of the 1-KB direct-to-LDS loads of one operand tile
// (R rows along M or N, one BK slice).  q0/qstep select the instructions.
template <int R, bool KMAJ>
__device__ __forceinline__ void load_tile(const OperandArgs& op, int64_t boff, int mn0, int k0,
                                          char LL_LDS* dst, int q0, int qstep, int lane) {
  const int64_t base = KMAJ ? boff + (int64_t)mn0 * op.ld + k0 : boff + (int64_t)k0 * op.ld + mn0;
  const i32x4 rsrc = make_rsrc(op.ptr + base, clamp_records(op.extent - base));
  constexpr int NQ = R / 8;
  const int ld = (int)op.ld;
  const uint32_t dst0 = lds_u32(dst);
#pragma unroll
  for (int q = q0; q < NQ; q += qstep) {
    uint32_t voff;
    if (KMAJ) {
      const int row = q * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ swz_k(row);
      const bool ok = (mn0 + row < op.rows) && (k0 + lc * 8 < op.kvalid);
      voff = ok ? (uint32_t)(row * ld + lc * 8) * 2u : kOOB;
    } else {
      constexpr int CH = R / 8;
      const int lin = q * 64 + lane;
      const int kr = lin / CH;
      const int lc = (lin % CH) ^ swz_mn<CH>(kr);
      const bool ok = (k0 + kr < op.kvalid) && (mn0 + lc * 8 < op.rows);
      voff = ok ? (uint32_t)(kr * ld + lc * 8) * 2u : kOOB;
    }
    dma16(rsrc, __builtin_amdgcn_readfirstlane(dst0 + q * 1024), voff);
  }
}

// Workgroup barrier ordering LDS only (global stores in flight are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// MFMA operand fragment: lane l holds rows/cols (r0 + l%32) and k = kk*16 + 8*(l/32) + j, j<8.
template <int R>
__device__ __forceinline__ bf16x8 frag_kmajor(const char LL_LDS* tile, int r0, int kk, int lane) {
  const int row = r0 + (lane & 31);
  const int lc = kk * 2 + (lane >> 5);
  return *(const bf16x8 LL_LDS*)(tile + row * 128 + ((lc ^ swz_k(row)) << 4));
}

// Same fragment from an MN-major tile.  ds_read_b64_tr_b16 gives lane i of each
// 16-lane group element i%4 of the 8-byte rows addressed by source lanes
// 4e + i/4 (e = 0..3): source lanes are pointed at k-rows so that element e
// is k-row e of the group, at column r0 + l%32.
template <int R>
__device__ __forceinline__ bf16x8 frag_mnmajor(const char LL_LDS* tile, int c0, int kk, int lane) {
  constexpr int CH = R / 8;
  const int g = lane >> 4, s = lane & 15;
  const int mn = c0 + 16 * (g & 1) + 4 * (s & 3);
  const int kr = kk * 16 + 8 * (g >> 1) + (s >> 2);
  const int lc = mn >> 3, half = (mn & 7) * 2;
  const char LL_LDS* p0 = tile + kr * (R * 2) + ((lc ^ swz_mn<CH>(kr)) << 4) + half;
  const char LL_LDS* p1 = tile + (kr + 4) * (R * 2) + ((lc ^ swz_mn<CH>(kr + 4)) << 4) + half;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LL_LDS*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LL_LDS*)p1);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

struct TileInfo {
  int b, ks, m0, n0, kb, ke;
};

template <int BM, int BN>
__device__ __forceinline__ TileInfo decode_tile(const GemmKArgs& p, int t) {
  const int tiles = p.tiles_m * p.tiles_n;
  const int tin = t % tiles;
  const int rest = t / tiles;
  TileInfo ti;
  ti.ks = rest % p.splits;
  ti.b = rest / p.splits;
  const int per_group = p.group_m * p.tiles_n;
  const int gid = tin / per_group;
  const int first_m = gid * p.group_m;
  const int gsz = min(p.tiles_m - first_m, p.group_m);
  const int w = tin - gid * per_group;
  ti.m0 = (first_m + w % gsz) * BM;
  ti.n0 = (w / gsz) * BN;
  ti.kb = ti.ks * p.kps;
  ti.ke = min(ti.kb + p.kps, p.kiters);
  return ti;
}

// Workgroup ids are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of work items so that tiles sharing A/B panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  if ((grid & 7) != 0) return bid;
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

template <int BM, int BN>
struct Cursor {
  int t, k;
  TileInfo ti;
  __device__ __forceinline__ void init(const GemmKArgs& p, int first) {
    t = first;
    if (t < p.total) {
      ti = decode_tile<BM, BN>(p, t);
      k = ti.kb;
    }
  }
  __device__ __forceinline__ bool valid(const GemmKArgs& p) const { return t < p.total; }
  __device__ __forceinline__ void advance(const GemmKArgs& p, int stride) {
    if (++k == ti.ke) {
      t += stride;
      if (t < p.total) {
        ti = decode_tile<BM, BN>(p, t);
        k = ti.kb;
      }
    }
  }
};

__device__ __forceinline__ int64_t batch_off(int b, int bdiv, int64_t bo, int64_t bi) {
  return (int64_t)(b / bdiv) * bo + (int64_t)(b % bdiv) * bi;
}

template <class Cfg>
__device__ __forceinline__ void issue_stage(const GemmKArgs& p, const TileInfo& ti, int k,
                                            char LL_LDS* slot, int lw, int lane) {
  const int k0 = k * kBK;
  load_tile<Cfg::BM, Cfg::A_KMAJOR>(p.a, batch_off(ti.b, p.bdiv, p.a.bo, p.a.bi), ti.m0, k0, slot,
                                    lw, Cfg::LOADERS, lane);
  load_tile<Cfg::BN, Cfg::B_KMAJOR>(p.b, batch_off(ti.b, p.bdiv, p.b.bo, p.b.bi), ti.n0, k0,
                                    slot + Cfg::A_BYTES, lw, Cfg::LOADERS, lane);
}

template <class Cfg>
__device__ __forceinline__ void load_frags(const char LL_LDS* slot, int kk, int wm0, int wn0, int lane,
                                           bf16x8 (&a)[Cfg::FM], bf16x8 (&b)[Cfg::FN]) {
  const char LL_LDS* sA = slot;
  const char LL_LDS* sB = slot + Cfg::A_BYTES;
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
    a[i] = Cfg::A_KMAJOR ? frag_kmajor<Cfg::BM>(sA, wm0 + 32 * i, kk, lane)
                         : frag_mnmajor<Cfg::BM>(sA, wm0 + 32 * i, kk, lane);
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    b[j] = Cfg::B_KMAJOR ? frag_kmajor<Cfg::BN>(sB, wn0 + 32 * j, kk, lane)
                         : frag_mnmajor<Cfg::BN>(sB, wn0 + 32 * j, kk, lane);
}

// One BK slice: four k16 steps; fragments of step kk+1 are requested before
// the MFMAs of step kk so that LDS latency overlaps matrix-core work.
template <class Cfg>
__device__ __forceinline__ void compute_stage(const char LL_LDS* slot, f32x16 (&acc)[Cfg::FM][Cfg::FN],
                                              int wm0, int wn0, int lane) {
  bf16x8 a[2][Cfg::FM], b[2][Cfg::FN];
  load_frags<Cfg>(slot, 0, wm0, wn0, lane, a[0], b[0]);
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < kBK / 16) load_frags<Cfg>(slot, kk + 1, wm0, wn0, lane, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: round to nearest even
}

// Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 block.
template <class Cfg>
__device__ __forceinline__ void epilogue(const GemmKArgs& p, const TileInfo& ti,
                                         const f32x16 (&acc)[Cfg::FM][Cfg::FN], int wm0, int wn0,
                                         int lane) {
  const int colb = ti.n0 + wn0 + (lane & 31);
  const int rowb = ti.m0 + wm0 + 4 * (lane >> 5);
  if (p.partial) {
    float* P = p.partial + (int64_t)ti.ks * p.M * p.N;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rowb + 32 * i + 8 * (r >> 2) + (r & 3);
          const int col = colb + 32 * j;
          if (row < p.M && col < p.N) P[(int64_t)row * p.N + col] = acc[i][j][r];
        }
    return;
  }
  const int64_t coff = batch_off(ti.b, p.bdiv, p.cbo, p.cbi);
  const int64_t boff = p.bias ? batch_off(ti.b, p.bdiv, p.bias_bo, p.bias_bi) : 0;
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int col = colb + 32 * j;
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = acc[i][j][r];
      if (p.bias) {
        float bv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rowb + 32 * i + 8 * (r >> 2) + (r & 3);
          bv[r] = (row < p.M && col < p.N) ? p.bias[boff + row * p.bias_m + col * p.bias_n] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += bv[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rowb + 32 * i + 8 * (r >> 2) + (r & 3);
        if (row < p.M && col < p.N) {
          const int64_t o = coff + (int64_t)row * p.ldcm + (int64_t)col * p.ldcn;
          if (p.c_bf16)
            ((uint16_t*)p.c)[o] = f32_to_bf16_bits(v[r]);
          else
            ((float*)p.c)[o] = v[r];
        }
      }
    }
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_EU, Cfg::WAVES_PER_EU)))
    gemm_persistent(const GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::LDS];
  char LL_LDS* smem = (char LL_LDS*)smem_raw;
  constexpr int S = Cfg::STAGES;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool is_cons = Cfg::NPROD == 0 || wave < Cfg::NCONS;
  const bool is_prod = Cfg::NPROD == 0 || wave >= Cfg::NCONS;
  const int lw = Cfg::NPROD == 0 ? wave : wave - Cfg::NCONS;
  const int cw = is_cons ? wave : 0;
  const int wm0 = (cw / Cfg::WN) * (Cfg::BM / Cfg::WM);
  const int wn0 = (cw % Cfg::WN) * (Cfg::BN / Cfg::WN);

  const int stride = gridDim.x;
  const int first = xcd_remap(blockIdx.x, gridDim.x);
  Cursor<Cfg::BM, Cfg::BN> lc, cc;
  lc.init(p, first);
  cc.init(p, first);

  int issued = 0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if (lc.valid(p)) {
      if (is_prod) issue_stage<Cfg>(p, lc.ti, lc.k, smem + s * Cfg::SLOT, lw, lane);
      lc.advance(p, stride);
      ++issued;
    }
  }

  f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bool drain = false;  // this wave issued global stores since its last full wait
  int j = 0;
  while (cc.valid(p)) {
    const int slot = j % S;
    if (is_prod) {
      if (!drain && issued - j - 1 >= S - 2)
        wait_vmcnt<(S - 2) * Cfg::LPW>();
      else
        wait_vmcnt<0>();
      drain = false;
    }
    lds_barrier();
    if (lc.valid(p)) {
      if (is_prod) issue_stage<Cfg>(p, lc.ti, lc.k, smem + ((j + S - 1) % S) * Cfg::SLOT, lw, lane);
      lc.advance(p, stride);
      ++issued;
    }
    if (is_cons) compute_stage<Cfg>(smem + slot * Cfg::SLOT, acc, wm0, wn0, lane);
    if (cc.k + 1 == cc.ti.ke) {
      if (is_cons) {
        epilogue<Cfg>(p, cc.ti, acc, wm0, wn0, lane);
        drain = true;
      }
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;
    }
    cc.advance(p, stride);
    ++j;
  }
}

}  // namespace ll
