// Persistent, software-pipelined bf16 GEMM for gfx950 (MI355X).
//
// What is computed: C = A.B (fp32 accumulation) over strided operands, as the
// listings on "Triton 3.7 permite extender el compilador de GPU sin forks"
// state the problem (sections "NVIDIA H100 (Hopper): GEMM persistente" and
// "AMD MI350: GEMM segmentado"), optionally split along K when the tiles
// alone cannot fill the chip.
//
// How (gfx950-specific design; the pages' TMA/WGMMA and register-staged
// mechanisms are not used):
//  * A ring of STAGES LDS slots.  Each slot holds one KT-deep k-slice of the
//    A tile and of the B tile.  Loading waves fill slots straight from HBM with
//    `buffer_load_dwordx4 ... lds` (no VGPR staging): each instruction moves
//    64 lanes x 16 B = 1 KB into a contiguous LDS block.  Lanes outside the
//    matrix get an offset beyond the buffer's num_records, so the hardware
//    writes zeros.
//  * Computing waves read MFMA operand fragments from LDS and run
//    v_mfma_f32_32x32x16_bf16.  A K-contiguous operand is stored [rows][KT]
//    (16-byte chunks XOR-swizzled by row) and read with ds_read_b128; an
//    M/N-contiguous operand is stored as it sits in memory, [KT][rows], and
//    read with ds_read_b64_tr_b16, which transposes 16-bit elements across
//    each group of 16 lanes.
//  * Handoff: one workgroup barrier per k-slice, placed before the slice's
//    last k16 step.  Before it, loading waves wait (vmcnt) until their share of
//    the NEXT slice has landed; after it, every wave has finished reading the
//    current slice's LDS (its last fragments are already in registers), so the
//    slice's slot is refilled at once and the next slice's first fragments are
//    read while the last k16 step's MFMAs run.  With NPROD > 0 the loading
//    and computing roles are separate waves; with NPROD == 0 every wave
//    computes and the first NLW waves (all if NLW == 0) also load.  The ring
//    runs across tile boundaries of the persistent loop.
//  * Persistent grid over (k-split, tile) work items in grouped
//    (GROUP_M) order, with workgroup ids remapped so that the consecutive
//    work items that share operand panels land on the same XCD (and its L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LL_LDS __attribute__((address_space(3)))

constexpr int kBK = 64;                    // k granularity the host plans in (largest KT)
constexpr uint32_t kOOB = 0x80000000u;     // byte offset beyond every num_records used here
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format

struct OperandArgs {
  const uint16_t* ptr;  // element (0, 0)
  int64_t ld;           // K-major: elements between MN rows; MN-major: elements between k rows
  int32_t rows;         // extent along M (A) or N (B)
  int32_t kvalid;       // k extent holding data; K-major operands: a multiple of 8
  int64_t extent;       // elements addressable from ptr (clamps num_records)
  int32_t once;         // each element is loaded by one work item only (non-temporal loads)
};

struct GemmKArgs {
  OperandArgs a, b;
  void* c;
  int64_t ldcm, ldcn;
  float* partial;     // split-K partials [splits][M][N], or null
  int32_t M, N;
  int32_t c_fmt;                // C elements: 0 fp32, 1 bf16, 2 fp16
  const float* bias;            // per-column addend (fp32, N values), or null
  int32_t act;                  // activation after the bias: 0 none, 1 ReLU, 2 GELU (erf form), 3 SiLU
  int32_t c_fast;               // 1: no partial, ldcn == 1, ldcm even, C 4-byte aligned (epilogue_fast)
  int32_t splits, kiters, kps;  // kiters, kps in units of KT
  int32_t tiles_m, tiles_n, group_m;
  int32_t total;
  // Hand-ordered kind only: per-XCD round counters (8 x 32 words, zeroed
  // before the launch), or null for no round barrier.
  uint32_t* sync;
  // Hand-ordered kind only: work items from tail_first on split the tiles of
  // a last round that would leave CUs idle tail_splits ways along K
  // (tail_kps slices each, the last split the rest) and leave raw fp32
  // partials in tail_partial ([item - tail_first][256][256]); a reduce
  // kernel finishes those tiles.  tail_first == total: no tail split.
  int32_t tail_first, tail_splits, tail_kps;
  float* tail_partial;
  // Hand-ordered kind only: 1 to prefetch the B slice after the next into
  // L2 (its loop always issues the prefetch; with 0 every lane's offset is
  // out of range and the load touches no memory).
  int32_t b_prefetch;
};

template <int BM_, int BN_, int KT_, int WM_, int WN_, int NPROD_, int STAGES_, bool AK_, bool BK_,
          bool F16_ = false, int EPI_ = 0, int NLW_ = 0>
struct GemmCfg {
  static constexpr bool F16 = F16_;           // A and B are fp16 (else bf16); same bytes, another MFMA
  // Fused epilogue, fixed per instantiation (a run-time choice among
  // activations costs the whole kernel its registers): 0 none; else the
  // per-column bias (if given) and activation EPI-1 (0 identity, 1 ReLU,
  // 2 GELU, 3 SiLU) on every sum before it is stored.
  static constexpr int EPI = EPI_;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int KT = KT_;              // k elements per ring slot (32 or 64)
  static constexpr int KS = KT / 16;          // k16 MFMA steps per slot
  static constexpr int WM = WM_, WN = WN_;    // computing-wave grid
  static constexpr int NCONS = WM * WN;
  static constexpr int NPROD = NPROD_;        // 0: every wave computes, and loads unless NLW says otherwise
  // With NPROD == 0: only waves 0 .. NLW-1 issue loads (0: every wave).  One
  // loading wave per SIMD leaves its partner wave free to run MFMAs while the
  // loading wave stalls issuing loads.
  static constexpr int NLW = NLW_;
  static constexpr int STAGES = STAGES_;
  static constexpr bool A_KMAJOR = AK_;       // A stored K-contiguous (row-major A)
  static constexpr bool B_KMAJOR = BK_;       // B stored K-contiguous (column-major B)
  static constexpr int WAVES = NCONS + NPROD;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // 32x32 blocks per wave
  static constexpr int A_BYTES = BM * KT * 2, B_BYTES = BN * KT * 2;
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGES * SLOT;
  static constexpr int LOADERS = NPROD ? NPROD : (NLW ? NLW : NCONS);
  static_assert(NLW == 0 || (NPROD == 0 && NLW <= NCONS), "loading subset of computing waves");
  static constexpr int QA = A_BYTES / 1024, QB = B_BYTES / 1024;  // 1-KB loads per slot
  static constexpr int LPW = (QA + QB) / LOADERS;                  // per loading wave
  static_assert(KT == 32 || KT == 64, "KT");
  static_assert(QA % LOADERS == 0 && QB % LOADERS == 0, "load split");
  static_assert(FM >= 1 && FN >= 1 && BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(STAGES >= 2, "stages");
  static_assert(LPW * (STAGES - 1) < 64, "vmcnt range");
  // An M/N-contiguous operand tile is loaded in 1-KB instructions that each
  // cover whole k-rows, so its width must divide 512 elements; kinds that
  // break this (a 192-row tile) exist only for K-contiguous operands.
  static constexpr bool VALID = (A_KMAJOR || 64 % (BM / 8) == 0) && (B_KMAJOR || 64 % (BN / 8) == 0);
  static constexpr int WAVES_PER_EU = (WAVES + 3) / 4;
  // Fragment buffers of a computing wave: two (the next k16 step's reads
  // overlap this step's MFMAs) unless accumulators plus two buffers would
  // not fit the wave's register budget (512 / waves per SIMD, less about 24
  // for addresses and loop state); then one, and the other computing waves
  // on the SIMD cover the LDS latency.
  static constexpr int FRAG_BUFS = FM * FN * 16 + 2 * 4 * (FM + FN) + 24 <= 512 / WAVES_PER_EU / 8 * 8 ? 2 : 1;
  static_assert(FM * FN * 16 <= 128 || WAVES_PER_EU == 1, "accumulators beyond 128 registers need the full file");
};

// ---------------------------------------------------------------------------
// LDS layouts.
//  K-major tile: [rows][KT] bf16, rows of CPR = KT/8 16-byte chunks; chunk c of
//  row r sits at c ^ swz_k(r).  For CPR = 8 the 8 (or 16) rows one
//  ds_read_b128 pass touches fall in distinct bank groups; for CPR = 4 (two
//  rows per 128-byte bank line) likewise for 8- and 16-lane passes.
//  MN-major tile: [KT][rows] bf16; chunk c of k-row r sits at c ^ swz_mn(r),
//  which spreads the 4 k-rows one ds_read_b64_tr_b16 lane group reads over
//  different banks.
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (CPR == 8) return (row ^ (row >> 3)) & 7;
  else return ((row >> 1) ^ (row >> 2)) & 3;
}
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
  r[3] = kRsrcWord3;
  return r;
}

// One direct-to-LDS load: lane l's 16 bytes at rsrc.base + voff land at LDS
// byte address m0 + 16*l.  Written as inline asm (M0 passed as an operand) so
// that the compiler does not order every later LDS access and barrier behind
// it with s_waitcnt vmcnt(0); completion is tracked by the explicit vmcnt
// waits of the pipeline instead.
//
// The compiler does not see a vector-memory instruction inside the asm, so it
// cannot pad the gfx9 hazards in front of it: a VALU write of an SGPR
// (v_readfirstlane building the descriptor, v_readlane restoring a spilled
// SGPR) needs 5 wait states before a VMEM instruction reads that SGPR, and an
// SALU write of M0 needs 1 before an LDS-DMA load.  The s_nop 4 covers both.
template <bool NT = false>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  if constexpr (NT)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const char LL_LDS* p) { return (uint32_t)(uintptr_t)p; }

// One direct-to-LDS load with a wave-uniform byte offset added (soffset);
// same hazard padding as dma16.  NT marks data that is read once (the
// non-temporal cache hint), so that it does not displace reused data in L2.
template <bool NT = false>
__device__ __forceinline__ void dma16s(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  if constexpr (NT)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}

// Issue this wave's share of the 1-KB direct-to-LDS loads of one operand tile
// (R rows along M or N, one KT slice): instructions q = lw, lw + NL, ...
//
// Instruction q covers tile rows (K-major) or k-rows (MN-major) q*RPQ ..
// q*RPQ + RPQ - 1.  In the fast path its byte offset splits into a
// wave-uniform part (slice offset + q*RPQ*ld*2, passed as soffset) and a
// per-lane part that depends on q only through q mod PER, the period of the
// swizzle pattern, so one or two offset registers serve all instructions.
// Tiles that reach past the matrix (last row/column tile, a k tail) take the
// masked path, where lanes outside the matrix get an offset beyond
// num_records and the hardware writes zeros.
template <int R, int KT, bool KMAJ>
struct TileGeom {
  static constexpr int NQ = R * KT * 2 / 1024;   // 1-KB instructions per tile
  static constexpr int CPR = KT / 8;             // K-major: 16-byte chunks per row
  static constexpr int CH = R / 8;               // MN-major: 16-byte chunks per k-row
  static constexpr int RPQ = KMAJ ? 64 / CPR : 64 / CH;
  static constexpr int PER = KMAJ ? (CPR == 8 ? 8 : 1) : (RPQ >= 4 ? 1 : 4 / RPQ);
  static_assert(KMAJ || (CH <= 64 && 64 % CH == 0), "MN-major tile rows must split a 1-KB load evenly");
  // Per-lane byte offset of instruction q (q mod PER) relative to its first row.
  __device__ static __forceinline__ uint32_t lane_off(int q, int lane, int ld) {
    const int qq = PER == 1 ? 0 : q % PER;
    int rl, lc;
    if constexpr (KMAJ) {
      rl = lane / CPR;
      lc = (lane % CPR) ^ swz_k<CPR>(qq * RPQ + rl);
    } else {
      rl = lane / CH;
      lc = (lane % CH) ^ swz_mn<CH>(qq * RPQ + rl);
    }
    return (uint32_t)(rl * ld + lc * 8) * 2u;
  }
};

template <int R, int KT, bool KMAJ, int NL, class Stream, bool NT = false>
__device__ __forceinline__ void load_tile(const OperandArgs& op, const Stream& o, bool fast, int mn0, int k0,
                                          char LL_LDS* dst, int lw, int lane, uint32_t vfast) {
  using G = TileGeom<R, KT, KMAJ>;
  static_assert(G::NQ % NL == 0, "load split");
  const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_u32(dst));
  const int ld = (int)op.ld;
  if (fast) {
#pragma unroll
    for (int i = 0; i < G::NQ / NL; ++i) {
      const int q = lw + i * NL;
      // vfast is lane_off(lw); other residues are recomputed (PER > NL only).
      const uint32_t voff = (NL % G::PER == 0) ? vfast : G::lane_off(q, lane, ld);
      const uint32_t soff = o.soff + (uint32_t)(q * G::RPQ) * (uint32_t)ld * 2u;
      dma16s<NT>(o.rs, dst0 + q * 1024, voff, soff);
    }
  } else {
    // Lanes outside the matrix: offset beyond num_records (the whole offset
    // sits in voff here, soffset is 0, so it cannot wrap back into range).
    // The empty asm makes the lane index opaque, so that these per-load
    // offsets (used only for tiles at the matrix edge) are computed here
    // rather than hoisted out of the main loop, where they held a dozen
    // registers for its whole length and made the 256x256 kind spill.
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int i = 0; i < G::NQ / NL; ++i) {
      const int q = lw + i * NL;
      uint32_t voff;
      if constexpr (KMAJ) {
        const int row = q * G::RPQ + lane / G::CPR;
        const int lc = (lane % G::CPR) ^ swz_k<G::CPR>(row);
        const bool ok = (mn0 + row < op.rows) && (k0 + lc * 8 < op.kvalid);
        voff = ok ? o.soff + (uint32_t)(row * ld + lc * 8) * 2u : kOOB;
      } else {
        const int lin = q * 64 + lane;
        const int kr = lin / G::CH;
        const int lc = (lin % G::CH) ^ swz_mn<G::CH>(kr);
        const bool ok = (k0 + kr < op.kvalid) && (mn0 + lc * 8 < op.rows);
        voff = ok ? o.soff + (uint32_t)(kr * ld + lc * 8) * 2u : kOOB;
      }
      dma16<NT>(o.rs, dst0 + q * 1024, voff);
    }
  }
}

// Workgroup barrier ordering LDS only (global stores in flight are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// MFMA operand fragment: lane l holds rows/cols (r0 + l%32) and k = kk*16 + 8*(l/32) + j, j<8.
template <int KT>
__device__ __forceinline__ bf16x8 frag_kmajor(const char LL_LDS* tile, int r0, int kk, int lane) {
  constexpr int CPR = KT / 8;
  const int row = r0 + (lane & 31);
  const int lc = kk * 2 + (lane >> 5);
  return *(const bf16x8 LL_LDS*)(tile + row * (KT * 2) + ((lc ^ swz_k<CPR>(row)) << 4));
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
  int ks, m0, n0, kb, ke;
};

// Tile tin (0 .. tiles_m * tiles_n - 1) in grouped order: groups of group_m
// tile rows, column by column within a group.
__device__ __forceinline__ void grouped_tile(int tin, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int gid = tin / per_group;
  const int first_m = gid * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int w = tin - gid * per_group;
  tm = first_m + w % gsz;
  tn = w / gsz;
}

template <class Cfg>
__device__ __forceinline__ TileInfo decode_tile(const GemmKArgs& p, int t) {
  const int tiles = p.tiles_m * p.tiles_n;
  const int tin = t % tiles;
  const int rest = t / tiles;
  TileInfo ti;
  ti.ks = rest;
  ti.kb = rest * p.kps;
  ti.ke = min(ti.kb + p.kps, p.kiters);
  int tm, tn;
  grouped_tile(tin, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  ti.m0 = tm * Cfg::BM;
  ti.n0 = tn * Cfg::BN;
  return ti;
}

// Workgroup ids are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of work items so that tiles sharing A/B panels share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  if ((grid & 7) != 0) return bid;
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

// Loading side of the pipeline.  Per operand: a buffer descriptor based at
// the work item's tile origin at slice `k0s` and a running wave-uniform byte
// offset along k, so that each slice costs one scalar add per operand.  The
// descriptor is re-based (opened again at the current slice) before the
// offset could leave the 32-bit range.
struct OpStream {
  i32x4 rs;
  uint32_t soff;  // byte offset of the next slice from the descriptor base
  int32_t k0s;    // slice (units of KT) at the descriptor base
};

template <class Cfg>
struct Loader {
  int t, k, ke;  // work item, next slice, end slice (units of KT)
  int m0, n0;
  bool rows_in;  // both operand tiles lie inside the matrix along M and N
  OpStream a, bo;

  template <int R, bool KMAJ>
  __device__ static __forceinline__ void open(OpStream& o, const OperandArgs& op, int mn0, int ks) {
    const int64_t origin = KMAJ ? (int64_t)mn0 * op.ld + (int64_t)ks * Cfg::KT
                                : (int64_t)ks * Cfg::KT * op.ld + mn0;
    o.rs = make_rsrc(op.ptr + origin, clamp_records(op.extent - origin));
    o.soff = 0;
    o.k0s = ks;
  }

  __device__ __forceinline__ void start(const GemmKArgs& p, int t_) {
    t = t_;
    if (t >= p.total) return;
    const TileInfo ti = decode_tile<Cfg>(p, t);
    k = ti.kb;
    ke = ti.ke;
    m0 = ti.m0;
    n0 = ti.n0;
    rows_in = m0 + Cfg::BM <= p.a.rows && n0 + Cfg::BN <= p.b.rows;
    open<Cfg::BM, Cfg::A_KMAJOR>(a, p.a, m0, k);
    open<Cfg::BN, Cfg::B_KMAJOR>(bo, p.b, n0, k);
  }

  __device__ __forceinline__ bool valid(const GemmKArgs& p) const { return t < p.total; }

  // Issue this wave's share of slice k into `slot`.
  __device__ __forceinline__ void issue(const GemmKArgs& p, char LL_LDS* slot, int lw, int lane, uint32_t va,
                                        uint32_t vb) const {
    const int k0 = k * Cfg::KT;
    // The two operands' k extents differ when one is a packed K-contiguous
    // copy (zero columns up to K rounded to 8) and the other is read in place
    // (exactly K): the unmasked path is taken only where both hold the slice.
    const bool fast = rows_in && k0 + Cfg::KT <= min(p.a.kvalid, p.b.kvalid);
    // an operand read by one work item only (one tile row or column) is
    // streamed with the non-temporal hint, so it does not push reused data
    // out of L2 (uniform branch)
    if (p.a.once)
      load_tile<Cfg::BM, Cfg::KT, Cfg::A_KMAJOR, Cfg::LOADERS, OpStream, true>(p.a, a, fast, m0, k0, slot, lw, lane,
                                                                             va);
    else
      load_tile<Cfg::BM, Cfg::KT, Cfg::A_KMAJOR, Cfg::LOADERS>(p.a, a, fast, m0, k0, slot, lw, lane, va);
    if (p.b.once)
      load_tile<Cfg::BN, Cfg::KT, Cfg::B_KMAJOR, Cfg::LOADERS, OpStream, true>(p.b, bo, fast, n0, k0,
                                                                             slot + Cfg::A_BYTES, lw, lane, vb);
    else
      load_tile<Cfg::BN, Cfg::KT, Cfg::B_KMAJOR, Cfg::LOADERS>(p.b, bo, fast, n0, k0, slot + Cfg::A_BYTES, lw,
                                                                lane, vb);
  }

  __device__ __forceinline__ void advance(const GemmKArgs& p, int stride) {
    if (++k == ke) {
      start(p, t + stride);
      return;
    }
    a.soff += Cfg::A_KMAJOR ? Cfg::KT * 2u : (uint32_t)(Cfg::KT * 2) * (uint32_t)p.a.ld;
    bo.soff += Cfg::B_KMAJOR ? Cfg::KT * 2u : (uint32_t)(Cfg::KT * 2) * (uint32_t)p.b.ld;
    if (a.soff >= (1u << 30)) open<Cfg::BM, Cfg::A_KMAJOR>(a, p.a, m0, k);
    if (bo.soff >= (1u << 30)) open<Cfg::BN, Cfg::B_KMAJOR>(bo, p.b, n0, k);
  }
};

template <class Cfg>
struct Frags {
  bf16x8 a[Cfg::FM], b[Cfg::FN];
};

template <class Cfg>
__device__ __forceinline__ void load_frags(const char LL_LDS* slot, int kk, int wm0, int wn0, int lane,
                                           Frags<Cfg>& f) {
  const char LL_LDS* sA = slot;
  const char LL_LDS* sB = slot + Cfg::A_BYTES;
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
    f.a[i] = Cfg::A_KMAJOR ? frag_kmajor<Cfg::KT>(sA, wm0 + 32 * i, kk, lane)
                           : frag_mnmajor<Cfg::BM>(sA, wm0 + 32 * i, kk, lane);
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j)
    f.b[j] = Cfg::B_KMAJOR ? frag_kmajor<Cfg::KT>(sB, wn0 + 32 * j, kk, lane)
                           : frag_mnmajor<Cfg::BN>(sB, wn0 + 32 * j, kk, lane);
}

// One 32x32x16 MFMA with fp32 accumulation; the fragments hold bf16 or, for
// F16, fp16 bit patterns (the LDS path moves 16-bit elements either way).
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One k16 step over the wave's FM x FN blocks of 32x32 (the accumulators are
// cleared separately when a tile starts).
template <class Cfg>
__device__ __forceinline__ void mfma_step(const Frags<Cfg>& f, f32x16 (&acc)[Cfg::FM][Cfg::FN]) {
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
      acc[i][j] = mfma32<Cfg::F16>(f.a[i], f.b[j], acc[i][j]);
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // v_cvt_pk_bf16_f32: round to nearest even
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  // The fp32 value is what gets rounded: without the empty asm the compiler
  // may fold a multiply before it into v_fma_mixlo_f16, which rounds the
  // exact product to fp16 once, and one sum would then differ by an ulp
  // between kernels and store paths.
  asm("" : "+v"(v));
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // v_cvt_f16_f32: round to nearest even
}

// erf(|x| / sqrt 2) by the rational approximation of Abramowitz and Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (absolute error at most
// 1.5e-7): erf(u) = 1 - (a1 t + ... + a5 t^5) exp(-u^2), t = 1 / (1 + p u),
// here with u = |x| / sqrt 2 folded into the constants: t = 1 / (1 + (p /
// sqrt 2) |x|) and exp(-u^2) = 2^(x^2 * (-log2(e) / 2)).  Branch free, so
// that an unrolled epilogue over every accumulator stays compact.  The
// reciprocal and the power of two are the hardware's (v_rcp_f32,
// v_exp_f32: about 1 ulp, no range handling), far inside the formula's own
// error; a correctly rounded reciprocal and a denormal-safe exp cost a dozen
// more vector operations per element, which with one wave per SIMD nothing
// hides.  Every multiply and add is spelled out (fmaf, __fmul_rn, __fadd_rn):
// left to the compiler, whether a product is fused into an add depends on
// the code around it, and the same sum would round differently in different
// kernels and store paths.
__device__ __forceinline__ float erf_as_scaled(float x) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.231641900f, fabsf(x), 1.f));  // 0.3275911 / sqrt 2
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float poly = __fmul_rn(t, q);
  const float g = __builtin_amdgcn_exp2f(__fmul_rn(__fmul_rn(x, x), -0.721347520f));  // exp(-x^2 / 2)
  return fmaf(-poly, g, 1.f);
}

// Epilogue arithmetic on one fp32 sum z plus its column's bias b: the
// activation ACT of z + b, in fp32.  GELU is the exact form z * Phi(z) =
// z/2 (1 + erf(z / sqrt 2)), as the product of z/2 and 1 + erf (exact where
// erf is near -1), which keeps the sign of z where the result underflows;
// SiLU z / (1 + exp(-z)) (exp(-z) = 2^(-z log2(e)); its overflow for very
// negative z gives the limit, -0).
template <int ACT>
__device__ __forceinline__ float epi(float z, float b) {
  const float x = __fadd_rn(z, b);
  if constexpr (ACT == 1) {
    return x > 0.f ? x : 0.f;
  } else if constexpr (ACT == 2) {
    const float e = erf_as_scaled(x);
    return __fmul_rn(__fmul_rn(0.5f, x), __fadd_rn(1.f, copysignf(e, x)));
  } else if constexpr (ACT == 3) {
    const float g = __builtin_amdgcn_exp2f(__fmul_rn(x, -1.442695041f));
    return __fmul_rn(x, __builtin_amdgcn_rcpf(__fadd_rn(1.f, g)));
  } else {
    return x;
  }
}

__device__ __forceinline__ float bias_at(const GemmKArgs& p, int col) { return p.bias ? p.bias[col] : 0.f; }

// 16-bit C element: bf16 (fmt 1) or fp16 (fmt 2), rounded to nearest even.
template <int FMT>
__device__ __forceinline__ uint16_t to_c16(float v) {
  if constexpr (FMT == 2) return f32_to_f16_bits(v);
  else return f32_to_bf16_bits(v);
}

// Swap with the neighbouring lane (lane ^ 1) via DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float swap_pair(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF,
                                                               false));
}

// Epilogue for a tile that lies wholly inside C, with C row-major
// (ldcn == 1) and no split-K.  Row bases are wave-uniform (scalar
// registers); each lane keeps one 32-bit element offset.  bf16 C: the lane
// pair holding columns d, d+1 swaps values so that each lane writes one
// 4-byte (d, d+1) pair per row - whole 128-byte lines, half the stores.
template <class Cfg, int FMT>
__device__ __forceinline__ void epilogue_fast16(const GemmKArgs& p, const TileInfo& ti,
                                                const f32x16 (&acc)[Cfg::FM][Cfg::FN], int wm0, int wn0,
                                                int lane) {
  const int row0 = ti.m0 + wm0;  // wave-uniform
  const int half = lane >> 5;
  const bool odd = lane & 1;
  const int col = ti.n0 + wn0 + (lane & 30);
  // lane-dependent part: row offset 4*half (+2 for the odd lane), column
  const int loff = (4 * half + (odd ? 2 : 0)) * (int)p.ldcm + col;
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint16_t* rowp = (uint16_t*)p.c + (int64_t)(row0 + 32 * i + 8 * g) * p.ldcm;
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) {
        const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        // the even lane sends rows 2, 3 and receives the odd lane's rows 0, 1
        // (column d+1); the odd lane sends rows 0, 1 and receives rows 2, 3
        const float s0 = swap_pair(odd ? v0 : v2);
        const float s1 = swap_pair(odd ? v1 : v3);
        const float a0 = odd ? s0 : v0, a1 = odd ? v2 : s0;
        const float b0 = odd ? s1 : v1, b1 = odd ? v3 : s1;
        const uint32_t pa = (uint32_t)to_c16<FMT>(a0) | ((uint32_t)to_c16<FMT>(a1) << 16);
        const uint32_t pb = (uint32_t)to_c16<FMT>(b0) | ((uint32_t)to_c16<FMT>(b1) << 16);
        *(uint32_t*)(rowp + loff + 32 * j) = pa;
        *(uint32_t*)(rowp + p.ldcm + loff + 32 * j) = pb;
      }
    }
}

// Epilogue for a tile that lies wholly inside C, with C row-major
// (ldcn == 1) and no split-K.  Row bases are wave-uniform (scalar
// registers); each lane keeps one 32-bit element offset.  16-bit C: the lane
// pair holding columns d, d+1 swaps values so that each lane writes one
// 4-byte (d, d+1) pair per row - whole 128-byte lines, half the stores.
template <class Cfg>
__device__ __forceinline__ void epilogue_fast(const GemmKArgs& p, const TileInfo& ti,
                                              const f32x16 (&acc)[Cfg::FM][Cfg::FN], int wm0, int wn0,
                                              int lane) {
  if (p.c_fmt == 1) {
    epilogue_fast16<Cfg, 1>(p, ti, acc, wm0, wn0, lane);
  } else if (p.c_fmt == 2) {
    epilogue_fast16<Cfg, 2>(p, ti, acc, wm0, wn0, lane);
  } else {
    const int row0 = ti.m0 + wm0;  // wave-uniform
    const int loff = 4 * (lane >> 5) * (int)p.ldcm + ti.n0 + wn0 + (lane & 31);
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float* rowp = (float*)p.c + (int64_t)(row0 + 32 * i + 8 * (r >> 2) + (r & 3)) * p.ldcm;
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) rowp[loff + 32 * j] = acc[i][j][r];
      }
  }
}

// Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 block.
template <class Cfg>
__device__ __forceinline__ void epilogue_any(const GemmKArgs& p, const TileInfo& ti,
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
          const float v = acc[i][j][r];
          if (row < p.M && col < p.N) P[(int64_t)row * p.N + col] = v;
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int col = colb + 32 * j;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rowb + 32 * i + 8 * (r >> 2) + (r & 3);
        const float v = acc[i][j][r];
        if (row < p.M && col < p.N) {
          const int64_t o = (int64_t)row * p.ldcm + (int64_t)col * p.ldcn;
          if (p.c_fmt == 1)
            ((uint16_t*)p.c)[o] = f32_to_bf16_bits(v);
          else if (p.c_fmt == 2)
            ((uint16_t*)p.c)[o] = f32_to_f16_bits(v);
          else
            ((float*)p.c)[o] = v;
        }
      }
    }
}

// The fast path needs: no split-K partial, unit column stride, the tile
// inside C, and (bf16) 4-byte aligned column pairs, i.e. an even row stride
// and an even base offset.  p.c_fast carries the host's check of the
// stride/alignment conditions.
// Bias and activation, in place on the accumulators before the store (the
// accumulators are cleared after the epilogue anyway).  Columns past N take
// no bias (those elements are not stored).
template <class Cfg, int ACT>
__device__ __forceinline__ void apply_epi(const GemmKArgs& p, const TileInfo& ti, f32x16 (&acc)[Cfg::FM][Cfg::FN],
                                          int wn0, int lane) {
#pragma unroll
  for (int j = 0; j < Cfg::FN; ++j) {
    const int col = ti.n0 + wn0 + (lane & 31) + 32 * j;
    const float b = col < p.N ? bias_at(p, col) : 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = epi<ACT>(acc[i][j][r], b);
  }
}

// Split-K partials stay raw sums (the reduce applies bias and activation).
template <class Cfg>
__device__ __forceinline__ void epilogue(const GemmKArgs& p, const TileInfo& ti, f32x16 (&acc)[Cfg::FM][Cfg::FN],
                                         int wm0, int wn0, int lane) {
  if constexpr (Cfg::EPI > 0) {
    if (!p.partial) apply_epi<Cfg, Cfg::EPI - 1>(p, ti, acc, wn0, lane);
  }
  if (p.c_fast && ti.m0 + Cfg::BM <= p.M && ti.n0 + Cfg::BN <= p.N)
    epilogue_fast<Cfg>(p, ti, acc, wm0, wn0, lane);
  else
    epilogue_any<Cfg>(p, ti, acc, wm0, wn0, lane);
}

// s_waitcnt vmcnt(n * LPW) for a wave-uniform 0 <= n < STAGES (n >= MAX
// waits for MAX * LPW): the wave's loads of the n slices issued after the
// one waited for may stay in flight.
template <class Cfg, int MAX>
__device__ __forceinline__ void wait_slices_upto(int n) {
  if constexpr (MAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAX) wait_vmcnt<MAX * Cfg::LPW>();
    else wait_slices_upto<Cfg, MAX - 1>(n);
  }
}
template <class Cfg>
__device__ __forceinline__ void wait_slices(int n) {
  wait_slices_upto<Cfg, Cfg::STAGES - 1>(n);
}

// Compute-side position in the workgroup's sequence of slices.
template <class Cfg>
struct CompPos {
  int ct, ck;  // work item, slice
  TileInfo ti;
  __device__ __forceinline__ void start(const GemmKArgs& p, int first) {
    ct = first;
    ti = decode_tile<Cfg>(p, ct);
    ck = ti.kb;
  }
  __device__ __forceinline__ bool tile_end() const { return ck + 1 == ti.ke; }
  __device__ __forceinline__ bool has_next(const GemmKArgs& p, int stride) const {
    return !tile_end() || ct + stride < p.total;
  }
  __device__ __forceinline__ void advance(const GemmKArgs& p, int stride) {
    if (tile_end()) {
      ct += stride;
      ti = decode_tile<Cfg>(p, ct);
      ck = ti.kb;
    } else {
      ++ck;
    }
  }
};

// Loading role (separate loading waves): fill the ring, then per slice wait
// until the next slice has landed, meet the computing waves at the barrier
// and refill the slot they have just released.
template <class Cfg>
__device__ __forceinline__ void producer_loop(const GemmKArgs& p, char LL_LDS* smem, int first, int stride,
                                              int lw, int lane) {
  constexpr int S = Cfg::STAGES;
  const uint32_t va = TileGeom<Cfg::BM, Cfg::KT, Cfg::A_KMAJOR>::lane_off(lw, lane, (int)p.a.ld);
  const uint32_t vb = TileGeom<Cfg::BN, Cfg::KT, Cfg::B_KMAJOR>::lane_off(lw, lane, (int)p.b.ld);
  Loader<Cfg> ld;
  ld.start(p, first);
  int issued = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (ld.valid(p)) {
      ld.issue(p, smem + s * Cfg::SLOT, lw, lane, va, vb);
      ld.advance(p, stride);
      ++issued;
    }
  }
  wait_slices<Cfg>(issued - 1);
  lds_barrier();
  CompPos<Cfg> cc;
  cc.start(p, first);
  int j = 0, slot = 0;
  while (true) {
    const bool has_next = cc.has_next(p, stride);
    if (has_next) wait_slices<Cfg>(issued - j - 2);
    lds_barrier();
    if (ld.valid(p)) {
      ld.issue(p, smem + slot * Cfg::SLOT, lw, lane, va, vb);
      ld.advance(p, stride);
      ++issued;
    }
    if (!has_next) break;
    cc.advance(p, stride);
    ++j;
    slot = slot + 1 == S ? 0 : slot + 1;
  }
}

// Computing role (separate computing waves): fragments from LDS, MFMAs, and
// the epilogue; one barrier per slice, placed before its last k16 step.
// Fragments are double-buffered (the next k16 step's reads overlap this
// step's MFMAs) unless the configuration runs three waves per SIMD, where the
// register budget only allows one buffer and the second computing wave on
// the SIMD covers the LDS latency instead.
template <class Cfg>
__device__ __forceinline__ void consumer_loop(const GemmKArgs& p, char LL_LDS* smem, int first, int stride,
                                              int cw, int lane) {
  constexpr int S = Cfg::STAGES;
  constexpr int KS = Cfg::KS;
  constexpr int NB = Cfg::FRAG_BUFS;
  const int wm0 = (cw / Cfg::WN) * (Cfg::BM / Cfg::WM);
  const int wn0 = (cw % Cfg::WN) * (Cfg::BN / Cfg::WN);
  f32x16 acc[Cfg::FM][Cfg::FN];
  zero_acc(acc);
  Frags<Cfg> f[NB];
  lds_barrier();
  load_frags<Cfg>(smem, 0, wm0, wn0, lane, f[0]);
  CompPos<Cfg> cc;
  cc.start(p, first);
  int slot = 0;
  while (true) {
    char LL_LDS* cur = smem + slot * Cfg::SLOT;
    const bool tile_end = cc.tile_end();
    const bool has_next = cc.has_next(p, stride);
    const int nslot = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (NB == 2) {
        if (kk + 1 < KS) {
          load_frags<Cfg>(cur, kk + 1, wm0, wn0, lane, f[(kk + 1) & 1]);
        } else {
          lds_barrier();
          if (has_next) load_frags<Cfg>(smem + nslot * Cfg::SLOT, 0, wm0, wn0, lane, f[0]);
        }
        mfma_step<Cfg>(f[kk & 1], acc);
      } else {
        mfma_step<Cfg>(f[0], acc);
        if (kk + 1 < KS) {
          load_frags<Cfg>(cur, kk + 1, wm0, wn0, lane, f[0]);
        } else {
          lds_barrier();
          if (has_next) load_frags<Cfg>(smem + nslot * Cfg::SLOT, 0, wm0, wn0, lane, f[0]);
        }
      }
    }
    if (tile_end) {
      epilogue<Cfg>(p, cc.ti, acc, wm0, wn0, lane);
      zero_acc(acc);
    }
    if (!has_next) break;
    cc.advance(p, stride);
    slot = nslot;
  }
}

// Every wave computes; waves below Cfg::LOADERS also load their share of
// each slice (all of them unless Cfg::NLW picks a subset).  Waves that do not
// load never wait on vmcnt.
template <class Cfg>
__device__ __forceinline__ void coop_loop(const GemmKArgs& p, char LL_LDS* smem, int first, int stride, int wave,
                                          int lane) {
  constexpr int S = Cfg::STAGES;
  constexpr int KS = Cfg::KS;
  const int wm0 = (wave / Cfg::WN) * (Cfg::BM / Cfg::WM);
  const int wn0 = (wave % Cfg::WN) * (Cfg::BN / Cfg::WN);
  const uint32_t va = TileGeom<Cfg::BM, Cfg::KT, Cfg::A_KMAJOR>::lane_off(wave, lane, (int)p.a.ld);
  const uint32_t vb = TileGeom<Cfg::BN, Cfg::KT, Cfg::B_KMAJOR>::lane_off(wave, lane, (int)p.b.ld);
  const bool loader = wave < Cfg::LOADERS;  // wave-uniform
  Loader<Cfg> ld;
  ld.start(p, first);
  int issued = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (loader && ld.valid(p)) {
      ld.issue(p, smem + s * Cfg::SLOT, wave, lane, va, vb);
      ld.advance(p, stride);
      ++issued;
    }
  }
  if (loader) wait_slices<Cfg>(issued - 1);
  lds_barrier();

  f32x16 acc[Cfg::FM][Cfg::FN];
  zero_acc(acc);
  Frags<Cfg> f[2];
  load_frags<Cfg>(smem, 0, wm0, wn0, lane, f[0]);

  bool drain = false;  // this wave issued global stores since its last full wait
  int j = 0;           // slices consumed so far
  int slot = 0;        // ring slot of slice j
  CompPos<Cfg> cc;
  cc.start(p, first);
  while (true) {
    char LL_LDS* cur = smem + slot * Cfg::SLOT;
    const bool tile_end = cc.tile_end();
    const bool has_next = cc.has_next(p, stride);
    const int nslot = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 1 < KS) {
        load_frags<Cfg>(cur, kk + 1, wm0, wn0, lane, f[(kk + 1) & 1]);
      } else {
        // Slice boundary: slice j+1 must have landed; slice j's LDS is free.
        if (has_next && loader) {
          wait_slices<Cfg>(drain ? 0 : issued - j - 2);
          drain = false;
        }
        lds_barrier();
        if (loader && ld.valid(p)) {
          ld.issue(p, cur, wave, lane, va, vb);
          ld.advance(p, stride);
          ++issued;
        }
        if (has_next) load_frags<Cfg>(smem + nslot * Cfg::SLOT, 0, wm0, wn0, lane, f[0]);
      }
      mfma_step<Cfg>(f[kk & 1], acc);
    }
    if (tile_end) {
      epilogue<Cfg>(p, cc.ti, acc, wm0, wn0, lane);
      drain = true;
      zero_acc(acc);
    }
    if (!has_next) break;
    cc.advance(p, stride);
    ++j;
    slot = nslot;
  }
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_EU, Cfg::WAVES_PER_EU)))
    gemm_persistent(const GemmKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::LDS];
  char LL_LDS* smem = (char LL_LDS*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x;
  const int first = xcd_remap(blockIdx.x, gridDim.x);
  if (first >= p.total) return;  // uniform over the workgroup
  if constexpr (Cfg::NPROD > 0) {
    if (wave >= Cfg::NCONS)
      producer_loop<Cfg>(p, smem, first, stride, wave - Cfg::NCONS, lane);
    else
      consumer_loop<Cfg>(p, smem, first, stride, wave, lane);
  } else {
    coop_loop<Cfg>(p, smem, first, stride, wave, lane);
  }
}

}  // namespace ll
