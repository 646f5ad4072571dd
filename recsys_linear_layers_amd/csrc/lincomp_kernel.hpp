// Fused, persistent RecSys linear-compression kernel for gfx950 (MI355X).
//
// What is computed (page "Meta accélère un noyau GPU d'un facteur 4 avec TLX",
// sections "Comment le chargement des données gêne le calcul" and "Ce que
// signifie une accélération d'un facteur quatre"): for request r and
// candidate c the layer input is the request's user rows stacked above the
// candidate's item rows, X = [user[r]; item[r][c]], and the output is
// Y[r][c] = W^T . X.  The user rows are the same for every candidate of a
// request, so their product U[r] = W[0:Nu]^T . user[r] is formed once per
// request and reused, instead of once per candidate.
//
// How:
//  * Work item = (Mo tile, D tile, request, range of candidates).  Per item
//    the ring carries first the Nu/KT "user" slices (A = W[0:Nu] rows,
//    B = user[r]) and then Ni/KT slices per candidate (A = W[Nu:] rows,
//    B = item[r][c]).  The consumer waves keep U[r] in registers at the end
//    of the user slices and start every candidate's accumulators from it, so
//    U never goes through memory and is never rounded.
//    Without dedup (asked for, or user rows given per candidate) the user
//    slices of the current candidate are streamed before its item slices and
//    the accumulators start from zero (the stacked-input form).
//  * Loading waves (NPROD) only stream slices HBM -> LDS with direct-to-LDS
//    loads; computing waves only read fragments, run MFMAs and store Y.  The
//    two roles run separate loops that meet at one workgroup barrier per
//    slice, so the computing waves' global stores never enter the loading
//    waves' vmcnt and never stall the ring.
//  * bf16 Y is stored as bf16 pairs: a DPP swap between neighbouring lanes
//    gives each lane two adjacent d values, so every store instruction
//    writes whole 128-byte lines.
#pragma once

#include "gemm_kernel.hpp"

namespace ll {

struct LincompKArgs {
  const uint16_t* user;
  const uint16_t* item;
  const uint16_t* W;
  void* Y;
  int32_t su_r, su_c, su_n, si_r, si_c, si_n, sw_n, sy_r, sy_c, sy_m;  // element strides (< 2^31)
  int64_t user_extent, item_extent, w_extent;  // elements addressable from each base pointer
  int32_t R, C, Nu, Ni, D, Mo;
  int32_t tiles_m, tiles_n, chunk, nchunks;    // candidates per work item, work items per request
  int32_t nu_sl, ni_sl;                        // slices per user / per candidate phase (>= 1 for Ni)
  int32_t total;                               // work items
  int32_t y_bf16, dedup;
  int32_t y_stage;  // bf16 Y, base and strides multiples of 16 bytes: whole-tile stores go through LDS
  // Ragged requests (offsets != nullptr): C is the total candidate count, the
  // candidates of request r are offsets[r] .. offsets[r+1]-1 (global indices
  // into item and Y, whose request strides are 0), and the candidates are cut
  // into nranges equal contiguous ranges, one per work item (per output tile).
  const int64_t* offsets;
  int32_t nranges;
  // Fused epilogue: bias[m] (Mo fp32 values, 16-byte aligned) added to every
  // sum of compressed row m before the activation (LincompCfg::ACT); null: none.
  const float* bias;
};

template <int BM_, int BN_, int KT_, int WN_, int NPROD_, int STAGES_, int ACT_ = 0, bool BIAS_ = false>
struct LincompCfg {
  // activation on every sum (plus its row's bias, BIAS) before it is stored:
  // 0 none, 1 ReLU, 2 GELU (erf form), 3 SiLU
  static constexpr int ACT = ACT_;
  static constexpr bool BIAS = BIAS_;
  static constexpr int BM = BM_, BN = BN_, KT = KT_, KS = KT / 16;
  static constexpr int WM = 1, WN = WN_;
  static constexpr int NCONS = WN, NPROD = NPROD_, STAGES = STAGES_;
  static constexpr bool F16 = false;  // bf16 inputs
  static constexpr int WAVES = NCONS + NPROD, THREADS = WAVES * 64;
  static constexpr int FM = BM / 32, FN = BN / WN / 32;
  static constexpr bool A_KMAJOR = false, B_KMAJOR = false;  // W^T and X are both MN-major in LDS
  static constexpr int A_BYTES = BM * KT * 2, B_BYTES = BN * KT * 2;
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGES * SLOT;
  // bf16 Y leaves through a per-wave LDS image after the ring (lc_flush)
  // where the image fits: 64 columns (128-byte rows) per wave
  static constexpr int IMG = BM * (BN / WN) * 2;
  static constexpr bool STAGE_Y = BN / WN == 64 && LDS + NCONS * IMG <= 160 * 1024;
  static constexpr int LDS_ALL = LDS + (STAGE_Y ? NCONS * IMG : 0);
  static constexpr int LOADERS = NPROD;
  static constexpr int LPW = (A_BYTES + B_BYTES) / 1024 / NPROD;
  static constexpr int WAVES_PER_EU = (WAVES + 3) / 4;
  static_assert(NPROD > 0, "the fused kernel uses separate loading waves");
  static_assert((A_BYTES / 1024) % NPROD == 0 && (B_BYTES / 1024) % NPROD == 0, "load split");
  static_assert(LDS_ALL <= 160 * 1024, "LDS");
  static_assert(STAGES >= 2 && STAGES <= 8, "stages");
  static_assert(LPW * (STAGES - 1) < 64, "vmcnt range");
  static_assert(FM * FN * 16 * 2 <= 160, "accumulators + U must leave room for fragments");
};

// Position in a work item's slice sequence.  Both roles walk the same
// sequence with their own copy.
struct LcPos {
  int t;         // work item
  int r, c, c1;  // request, current candidate, end of the item's candidates
  int rend;      // end of the current request's candidates within the item
  int m0, n0;    // output tile origin (Mo, D)
  bool user;     // current slice belongs to the user phase
  int ks;        // slice index within the phase

  // offsets[q] clamped to [0, C]: malformed offsets give wrong rows, never an
  // access outside the buffers.
  __device__ static __forceinline__ int off_at(const LincompKArgs& p, int q) {
    const int64_t v = p.offsets[q];
    return (int)(v < 0 ? 0 : (v > p.C ? (int64_t)p.C : v));
  }
  // First candidate index >= c that starts a later request than r.
  __device__ __forceinline__ void next_request(const LincompKArgs& p) {
    while (r + 1 < p.R && off_at(p, r + 1) <= c) ++r;
    const int e = min(off_at(p, r + 1), c1);
    rend = e > c ? e : c + 1;  // progress even on malformed offsets
  }

  __device__ __forceinline__ void start(const LincompKArgs& p, int t_) {
    t = t_;
    if (t >= p.total) return;
    const int tiles = p.tiles_m * p.tiles_n;
    const int tin = t % tiles;
    const int rc = t / tiles;
    m0 = tin / p.tiles_n;  // tile indices along Mo and D
    n0 = tin - m0 * p.tiles_n;
    ks = 0;
    user = p.nu_sl > 0;
    if (p.offsets) {
      c = (int)((int64_t)rc * p.C / p.nranges);
      c1 = (int)((int64_t)(rc + 1) * p.C / p.nranges);
      // request of candidate c: the last r with offsets[r] <= c
      int lo = 0, hi = p.R - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off_at(p, mid) <= c) lo = mid;
        else hi = mid - 1;
      }
      r = lo;
      next_request(p);
      return;
    }
    r = rc / p.nchunks;
    const int ch = rc - r * p.nchunks;
    c = ch * p.chunk;
    c1 = min(c + p.chunk, p.C);
    rend = c1;
  }
  __device__ __forceinline__ bool valid(const LincompKArgs& p) const { return t < p.total; }
  // Last slice of the user phase (dedup: U is complete after it).
  __device__ __forceinline__ bool user_end(const LincompKArgs& p) const { return user && ks + 1 == p.nu_sl; }
  // Last slice of a candidate (its result is complete after it).
  __device__ __forceinline__ bool cand_end(const LincompKArgs& p) const { return !user && ks + 1 == p.ni_sl; }
  // Last slice of the request's candidates in this item (the next candidate,
  // if any, needs a new U).
  __device__ __forceinline__ bool req_end(const LincompKArgs& p) const { return cand_end(p) && c + 1 >= rend; }
  __device__ __forceinline__ bool item_end(const LincompKArgs& p) const { return cand_end(p) && c + 1 == c1; }
  __device__ __forceinline__ void advance(const LincompKArgs& p, int stride) {
    if (user) {
      if (++ks == p.nu_sl) {
        user = false;
        ks = 0;
      }
      return;
    }
    if (++ks < p.ni_sl) return;
    ks = 0;
    if (++c < c1) {
      if (c >= rend) {  // ragged: the next request starts
        next_request(p);
        user = p.nu_sl > 0;
      } else {
        user = !p.dedup && p.nu_sl > 0;
      }
      return;
    }
    start(p, t + stride);
  }
};

// Slice origin (elements from the base pointers) and operand descriptions for
// one slice.  rows/kvalid feed the masked path of load_tile.
struct SliceStream {
  i32x4 rs;
  uint32_t soff;
};

template <class Cfg>
__device__ __forceinline__ void lc_issue(const LincompKArgs& p, const LcPos& s, char LL_LDS* slot, int lw,
                                         int lane, uint32_t va, uint32_t vb) {
  const int k0 = s.ks * Cfg::KT;
  const int kvalid = s.user ? p.Nu : p.Ni;
  const int m0 = s.m0 * Cfg::BM, n0 = s.n0 * Cfg::BN;
  // A = W^T: A[m][n] = W[wrow0 + n][m], MN-major with ld = sw_n.
  OperandArgs oa;
  oa.ld = p.sw_n;
  oa.rows = p.Mo;
  oa.kvalid = kvalid;
  const int64_t wrow0 = s.user ? 0 : p.Nu;
  const int64_t aorg = (wrow0 + k0) * p.sw_n + m0;
  SliceStream sa;
  sa.rs = make_rsrc(p.W + aorg, clamp_records(p.w_extent - aorg));
  sa.soff = 0;
  // B = X rows: user[r] or item[r][c], MN-major with ld = su_n / si_n.
  OperandArgs ob;
  ob.rows = p.D;
  ob.kvalid = kvalid;
  SliceStream sb;
  sb.soff = 0;
  if (s.user) {
    ob.ld = p.su_n;
    const int64_t borg = (int64_t)s.r * p.su_r + (int64_t)s.c * p.su_c + (int64_t)k0 * p.su_n + n0;
    sb.rs = make_rsrc(p.user + borg, clamp_records(p.user_extent - borg));
  } else {
    ob.ld = p.si_n;
    const int64_t borg = (int64_t)s.r * p.si_r + (int64_t)s.c * p.si_c + (int64_t)k0 * p.si_n + n0;
    sb.rs = make_rsrc(p.item + borg, clamp_records(p.item_extent - borg));
  }
  const bool kin = k0 + Cfg::KT <= kvalid;
  const bool fa = kin && m0 + Cfg::BM <= p.Mo;
  const bool fb = kin && n0 + Cfg::BN <= p.D;
  load_tile<Cfg::BM, Cfg::KT, false, Cfg::LOADERS>(oa, sa, fa, m0, k0, slot, lw, lane, va);
  // user and item rows are read once: non-temporal hint
  load_tile<Cfg::BN, Cfg::KT, false, Cfg::LOADERS, SliceStream, true>(ob, sb, fb, n0, k0, slot + Cfg::A_BYTES, lw,
                                                                       lane, vb);
}

// Bias of the four compressed rows of a lane's group: rows m8 + 4 half ..
// + 3, where m8 (a multiple of 8, uniform over the wave) is the group's first
// row and half = lane / 32; zeros without a bias.  The eight values of rows
// m8 .. m8 + 7 come through scalar loads (the address is wave-uniform and the
// bias is read-only): a vector load here would count with the wave's Y
// stores, and waiting for it would wait for every store issued before it.
// Mo is a multiple of 8, so the eight rows are all in range or all out.
template <bool BIAS>
__device__ __forceinline__ f32x4 lc_bias4(const LincompKArgs& p, int m8, int half) {
  f32x4 b = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BIAS) {
    if (m8 < p.Mo) {
      typedef const float __attribute__((address_space(4)))* cptr;
      const cptr q = (cptr)(p.bias + m8);
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = q[k];
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = half ? v[4 + r] : v[r];
    }
  }
  return b;
}

// One group of a bf16 Y block: values v0..v3 of rows q%4 = 0..3 at this
// lane's column.  Lane pair (2i, 2i+1) holds columns d, d+1 of the same rows:
// the even lane sends rows 2, 3 and receives the odd lane's rows 0, 1
// (column d+1), the odd lane sends rows 0, 1 and receives rows 2, 3 (column
// d), and each lane stores the (d, d+1) pairs of its two rows.  Y + off is
// this lane's first row of the group (row ra) at column d; sym is the row
// stride.
__device__ __forceinline__ void lc_store_group(const LincompKArgs& p, uint16_t* Y, int off, int sym, int ra, int dd,
                                               bool odd, float v0, float v1, float v2, float v3) {
  const float s0 = swap_pair(odd ? v0 : v2);
  const float s1 = swap_pair(odd ? v1 : v3);
  float a0, a1, b0, b1;  // row ra: (a0 at d, a1 at d+1); row ra+1: (b0, b1)
  if (!odd) {
    a0 = v0; a1 = s0;
    b0 = v1; b1 = s1;
  } else {
    a0 = s0; a1 = v2;
    b0 = s1; b1 = v3;
  }
  const uint32_t pa = (uint32_t)f32_to_bf16_bits(a0) | ((uint32_t)f32_to_bf16_bits(a1) << 16);
  const uint32_t pb = (uint32_t)f32_to_bf16_bits(b0) | ((uint32_t)f32_to_bf16_bits(b1) << 16);
  if (dd < p.D) {  // D is a multiple of 8, so dd < D implies dd + 1 < D
    if (ra < p.Mo) *(uint32_t*)(Y + off) = pa;
    if (ra + 1 < p.Mo) *(uint32_t*)(Y + off + sym) = pb;
  }
}

// Staged bf16 Y: the wave's BM x 64 block goes into its own LDS image and
// back out in whole 128-byte lines, 16 bytes per lane (8 rows of a 64-column
// segment per store instruction instead of 4 half lines per instruction).
// The image has 128-byte rows; row q sits at physical row q ^ ((q >> 2) & 1)
// and its 16-byte chunk c at c ^ (((q >> 1) & 1) << 2).  A pair write covers
// rows 8k + {0,2,4,6} (or {1,3,5,7}) x 64 bytes: the four land in four
// different 64-byte bank windows of 256 bytes, and the two rows of each half
// wave in different halves of 128 bytes, so neither a 64-bank nor a 32-bank
// pass conflicts; a 16-byte read covers whole rows, two adjacent ones of
// opposite parity per 16 lanes.  Each wave only reads back what it wrote, in
// order, so no barrier is needed; the next candidate's writes follow this
// one's reads in the same wave.
__device__ __forceinline__ uint32_t lc_img_off(int q, int cb) {
  return (uint32_t)(((q ^ ((q >> 2) & 1)) << 7) + ((((cb >> 4) ^ (((q >> 1) & 1) << 2))) << 4) + (cb & 15));
}

// One group of staged values: v0..v3 of rows q%4 = 0..3 at this lane's
// column, lane-pair swapped as in lc_store_group; the pair of row q goes to
// LDS byte address wa, that of row q+1 to wb.
__device__ __forceinline__ void lc_stage_group(uint32_t wa, uint32_t wb, bool odd, float v0, float v1, float v2,
                                               float v3) {
  const float s0 = swap_pair(odd ? v0 : v2);
  const float s1 = swap_pair(odd ? v1 : v3);
  float a0, a1, b0, b1;  // row q: (a0 at d, a1 at d+1); row q+1: (b0, b1)
  if (!odd) {
    a0 = v0; a1 = s0;
    b0 = v1; b1 = s1;
  } else {
    a0 = s0; a1 = v2;
    b0 = s1; b1 = v3;
  }
  *(uint32_t LL_LDS*)(uintptr_t)wa = (uint32_t)f32_to_bf16_bits(a0) | ((uint32_t)f32_to_bf16_bits(a1) << 16);
  *(uint32_t LL_LDS*)(uintptr_t)wb = (uint32_t)f32_to_bf16_bits(b0) | ((uint32_t)f32_to_bf16_bits(b1) << 16);
}

// The image back, eight rows per 16-byte read, and out to Y (Yw: the wave's
// block origin, sym its row stride).  Rows 8k + rl keep the lane's physical
// row and chunk swizzle of row rl, so the reads step by 1 KB.
template <int BM>
__device__ __forceinline__ void lc_flush(uint16_t* Yw, int sym, int lane, uint32_t img) {
  const int rl = lane >> 3, c = lane & 7;
  const uint32_t ra = img + lc_img_off(rl, c * 16);
  int off = rl * sym + c * 8;
#pragma unroll 2
  for (int k = 0; k < BM / 8; ++k) {
    const i32x4 v = *(const i32x4 LL_LDS*)(uintptr_t)(ra + k * 1024);
    // Y is written once and not read again by this kernel: non-temporal
    // (with whole lines, 3-4% faster than cached stores of the same lines)
    __builtin_nontemporal_store(v, (i32x4*)(Yw + off));
    off += 8 * sym;
  }
}

// Stores the wave's FM x FN blocks of Y for candidate (r, c).  Accumulator
// layout of v_mfma_f32_32x32x16: register q of lane l holds row 8*(q/4) +
// 4*(l/32) + q%4, column l%32 of the 32x32 block.  The block is addressed
// from a wave-uniform base with one 32-bit element offset per lane (the host
// keeps Mo * sy_m below 2^30) and row steps that are wave-uniform multiples
// of sy_m.
//  * Plain layer: block after block, each group by group (storing the two
//    column blocks of a row group back to back was 9% slower on the 256 x 128
//    workload).
//  * Fused epilogue (each value's row bias, then the activation, four values
//    at a time just before they are rounded): group by group across the
//    column blocks, so that one 16-byte bias load serves the four rows of a
//    group for every block and the activation's temporaries stay few.
template <class Cfg>
__device__ __forceinline__ void lc_epilogue(const LincompKArgs& p, const LcPos& s, f32x16 (&acc)[Cfg::FM][Cfg::FN],
                                            int wn0, int lane, char LL_LDS* img) {
  constexpr bool any_epi = Cfg::ACT != 0 || Cfg::BIAS;
  const int64_t yoff = (int64_t)s.r * p.sy_r + (int64_t)s.c * p.sy_c;
  const int sym = (int)p.sy_m;
  const int mb = s.m0 * Cfg::BM + 4 * (lane >> 5);
  const int db = s.n0 * Cfg::BN + wn0 + (lane & 31);
  // the wave's whole block inside Y, 16-byte aligned rows (p.y_stage: the
  // base and the strides are multiples of 16 bytes; wave-uniform)
  if (Cfg::STAGE_Y && p.y_stage && s.m0 * Cfg::BM + Cfg::BM <= p.Mo && s.n0 * Cfg::BN + wn0 + 64 <= p.D) {
    const bool odd = lane & 1;
    const int q0 = 4 * (lane >> 5) + (odd ? 2 : 0);  // this lane's first row, 0, 2, 4 or 6
    const int cb = 2 * (lane & 30);                   // byte of its column pair in a 64-column block
    const uint32_t im = lds_u32(img);
    // rows q0 + 32 i + 8 g (+1) keep the swizzle of rows q0 (+1): two base
    // addresses per column block, constant offsets per (i, g)
    uint32_t wa[Cfg::FN], wb[Cfg::FN];
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      wa[j] = im + lc_img_off(q0, cb + 64 * j);
      wb[j] = im + lc_img_off(q0 + 1, cb + 64 * j);
    }
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b = lc_bias4<Cfg::BIAS>(p, s.m0 * Cfg::BM + 32 * i + 8 * g, lane >> 5);
        const uint32_t ro = (32 * i + 8 * g) * 128;
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
          const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if constexpr (any_epi)
            lc_stage_group(wa[j] + ro, wb[j] + ro, odd, epi<Cfg::ACT>(v0, b[0]), epi<Cfg::ACT>(v1, b[1]),
                           epi<Cfg::ACT>(v2, b[2]), epi<Cfg::ACT>(v3, b[3]));
          else
            lc_stage_group(wa[j] + ro, wb[j] + ro, odd, v0, v1, v2, v3);
        }
      }
    lc_flush<Cfg::BM>((uint16_t*)p.Y + yoff + (int64_t)(s.m0 * Cfg::BM) * sym + s.n0 * Cfg::BN + wn0, sym, lane,
                      im);
    return;
  }
  if (p.y_bf16) {
    uint16_t* Y = (uint16_t*)p.Y + yoff;
    const bool odd = lane & 1;
    const int d = db - (lane & 1);
    const int r0 = mb + (odd ? 2 : 0);  // this lane's first row
    const int loff = r0 * sym + d;
    if constexpr (!any_epi) {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            lc_store_group(p, Y, loff + (32 * i + 8 * g) * sym + 32 * j, sym, r0 + 32 * i + 8 * g, d + 32 * j, odd,
                           acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 b = lc_bias4<Cfg::BIAS>(p, s.m0 * Cfg::BM + 32 * i + 8 * g, lane >> 5);
#pragma unroll
          for (int j = 0; j < Cfg::FN; ++j)
            lc_store_group(p, Y, loff + (32 * i + 8 * g) * sym + 32 * j, sym, r0 + 32 * i + 8 * g, d + 32 * j, odd,
                           epi<Cfg::ACT>(acc[i][j][4 * g], b[0]), epi<Cfg::ACT>(acc[i][j][4 * g + 1], b[1]),
                           epi<Cfg::ACT>(acc[i][j][4 * g + 2], b[2]), epi<Cfg::ACT>(acc[i][j][4 * g + 3], b[3]));
        }
    }
  } else {
    float* Y = (float*)p.Y + yoff;
    const int loff = mb * sym + db;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b = lc_bias4<Cfg::BIAS>(p, s.m0 * Cfg::BM + 32 * i + 8 * g, lane >> 5);
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = mb + 32 * i + 8 * g + r;
            const float v = any_epi ? epi<Cfg::ACT>(acc[i][j][4 * g + r], b[r]) : acc[i][j][4 * g + r];
            if (m < p.Mo && db + 32 * j < p.D) Y[loff + (32 * i + 8 * g + r) * sym + 32 * j] = v;
          }
      }
  }
}

// s_waitcnt vmcnt(min(n, MAX) * LPW) for a wave-uniform n >= 0: at most n
// slices of this wave's loads may stay in flight.
template <class Cfg, int MAX>
__device__ __forceinline__ void lc_wait_upto(int n) {
  if constexpr (MAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAX) wait_vmcnt<MAX * Cfg::LPW>();
    else lc_wait_upto<Cfg, MAX - 1>(n);
  }
}
template <class Cfg>
__device__ __forceinline__ void lc_wait(int n) {
  lc_wait_upto<Cfg, Cfg::STAGES - 1>(n);
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_EU, Cfg::WAVES_PER_EU)))
    lincomp_fused(const LincompKArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[Cfg::LDS_ALL];
  char LL_LDS* smem = (char LL_LDS*)smem_raw;
  constexpr int S = Cfg::STAGES;
  constexpr int KS = Cfg::KS;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x;
  const int first = xcd_remap(blockIdx.x, gridDim.x);
  if (first >= p.total) return;  // uniform over the workgroup

  if (wave >= Cfg::NCONS) {
    // ---------------- loading waves ----------------
    const int lw = wave - Cfg::NCONS;
    const uint32_t va = TileGeom<Cfg::BM, Cfg::KT, false>::lane_off(lw, lane, (int)p.sw_n);
    const uint32_t vbu = TileGeom<Cfg::BN, Cfg::KT, false>::lane_off(lw, lane, (int)p.su_n);
    const uint32_t vbi = TileGeom<Cfg::BN, Cfg::KT, false>::lane_off(lw, lane, (int)p.si_n);
    LcPos ld;
    ld.start(p, first);
    int issued = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (ld.valid(p)) {
        lc_issue<Cfg>(p, ld, smem + s * Cfg::SLOT, lw, lane, va, ld.user ? vbu : vbi);
        ld.advance(p, stride);
        ++issued;
      }
    }
    lc_wait<Cfg>(issued - 1);
    lds_barrier();
    int j = 0, slot = 0;
    while (true) {
      // slice j+1 exists if it was issued already or more slices are left
      const bool has_next = j + 1 < issued || ld.valid(p);
      if (has_next) lc_wait<Cfg>(issued - j - 2);
      lds_barrier();
      if (ld.valid(p)) {
        lc_issue<Cfg>(p, ld, smem + slot * Cfg::SLOT, lw, lane, va, ld.user ? vbu : vbi);
        ld.advance(p, stride);
        ++issued;
      }
      if (!has_next) break;
      ++j;
      slot = slot + 1 == S ? 0 : slot + 1;
    }
    return;
  }

  // ---------------- computing waves ----------------
  const int wn0 = wave * (Cfg::BN / Cfg::WN);
  char LL_LDS* img = smem + Cfg::LDS + (Cfg::STAGE_Y ? wave * Cfg::IMG : 0);
  f32x16 acc[Cfg::FM][Cfg::FN], u[Cfg::FM][Cfg::FN];
  zero_acc(acc);
  zero_acc(u);
  // One fragment buffer: the next k16 step's reads follow this step's MFMAs
  // (the computing waves are far from busy in this HBM-bound layer, and the
  // 32 VGPRs of a second buffer pushed the kernel into spilling).
  Frags<Cfg> f;
  lds_barrier();
  load_frags<Cfg>(smem, 0, 0, wn0, lane, f);
  LcPos cc;
  cc.start(p, first);
  int slot = 0;
  while (true) {
    char LL_LDS* cur = smem + slot * Cfg::SLOT;
    const bool item_end = cc.item_end(p);
    const bool has_next = !item_end || cc.t + stride < p.total;
    const int nslot = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      mfma_step<Cfg>(f, acc);
      if (kk + 1 < KS) {
        load_frags<Cfg>(cur, kk + 1, 0, wn0, lane, f);
      } else {
        lds_barrier();
        if (has_next) load_frags<Cfg>(smem + nslot * Cfg::SLOT, 0, 0, wn0, lane, f);
      }
    }
    if (p.dedup && cc.user_end(p)) {
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < Cfg::FN; ++jj) u[i][jj] = acc[i][jj];
    }
    if (cc.cand_end(p)) {
      lc_epilogue<Cfg>(p, cc, acc, wn0, lane, img);
      if (p.dedup && !cc.req_end(p)) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
          for (int jj = 0; jj < Cfg::FN; ++jj) acc[i][jj] = u[i][jj];
      } else {
        zero_acc(acc);
      }
    }
    if (item_end) {
      zero_acc(acc);
      zero_acc(u);
    }
    if (!has_next) break;
    cc.advance(p, stride);
    slot = nslot;
  }
}

}  // namespace ll
