// C ABI of liblinlayers.so: argument checks, plan selection (tile shape,
// wave roles, split-K, packing, grid), workspace layout and launches.
// The declarations and their contracts are in include/linlayers.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/linlayers.h"
#include "kernels.hpp"
#include "lincomp_kernel.hpp"

using namespace ll;

namespace {

thread_local std::string g_last_error;

ll_status fail(ll_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ll_status fail(ll_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ll_status ok() {
  g_last_error.clear();
  return LL_OK;
}

ll_status hip_fail(hipError_t e, const char* what) {
  return fail(LL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int cus = 0;
  char arch[64] = {0};
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// Current device, its CU count, and whether it is gfx950.
ll_status current_device(int* dev, const DeviceInfo** info) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) return fail(LL_ERR_NO_DEVICE, "no HIP device visible");
  e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (*dev < 0 || *dev >= 64) return fail(LL_ERR_UNSUPPORTED, "device index %d out of range", *dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[*dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, *dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.cus = prop.multiProcessorCount;
    snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.probed = true;
  }
  *info = &d;
  if (!d.gfx950) return fail(LL_ERR_UNSUPPORTED, "device %d is %s; this library targets gfx950", *dev, d.arch);
  return LL_OK;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The hand-ordered kind's tail split: at most this many K splits per tile of
// a last round that is at most half full, each of at least this many slices.
// Measured with and without it, same process: the edge shape (128 tiles, 2
// splits) +8.8%, 8448^2 x 4096 (65 x 3) +10.6%, 12288 x 4608 x 8192 (96 x
// 2) +8.9%, 4352 x 4096 x 4096 (16 x 4) +18.4%; with 8-slice splits
// (8448^2 x 1024) -3.6%, the partials' traffic outweighing the time saved.
constexpr int kTailMaxSplits = 4;
constexpr int kTailMinSlices = 16;

// K splits of the tail of a hand-ordered plan with `tiles` tiles on `grid`
// workgroups and `kiters` 64-deep slices: 1 (no tail split) unless there is
// a whole round and a last round at most half full.
int tail_splits_for(int64_t tiles, int64_t grid, int kiters) {
  if (grid <= 0 || tiles <= grid || kiters < 2 * kTailMinSlices) return 1;
  const int64_t last = tiles % grid;
  if (last == 0 || last * 2 > grid) return 1;
  const char* env = getenv("LL_GEMM_TAIL_SPLIT");
  if (env && env[0] == '0') return 1;
  int s = (int)std::min<int64_t>(std::min<int64_t>(grid / last, kTailMaxSplits), kiters / kTailMinSlices);
  if (s < 2) return 1;
  const int kps = (kiters + s - 1) / s;
  return (kiters + kps - 1) / kps;  // every split gets >= 1 slice (>= kTailMinSlices but the last)
}

// The hand-ordered kind's round counters: one per XCD, 128 bytes apart.
constexpr int kRoundSyncWords = 8 * 32;
// Fewest rounds (passes of the persistent grid over its tiles), and fewest
// 64-deep slices per tile, for which the plan turns the round barrier on.
// Measured with and without it, same process: FFN-up (28 rounds of 128
// slices) +4.9%, the same with bias + GELU +4.1%, FFN-down (8 of 448)
// +0.35%, 16384 x 8192 x 8192 (8 of 128) +0.1%; shorter tiles lose:
// 16384^2 x 4096 (16 of 64) -1.8%, 8192^2 x 4096 and 8192^3 (4) -1%,
// 8192^2 x 1024 (4 of 16) -7%, 4096 x 8192 x 8192 (2) -1.8%.  The drift it
// removes builds up over many long rounds; on short ones the wait costs more.
constexpr int kRoundSyncMinRounds = 8;
constexpr int kRoundSyncMinSlices = 128;

// The hand-ordered kind's L2 prefetch of B: on when B's rows (as the kernel
// reads them) are at least this many elements apart and tiles have at least
// this many slices.  Same process, with and without it: 8192 x 28672 x 8192
// +7.4%, FFN-up +6.9%, 16384 x 24576 x 8192 +5.4%, 16384^2 x 8192 and 8192 x
// 16384 x 8192 +0.7 to +0.9%; with K = 4096 -2 to +0.4%, FFN-down (B rows
// 8192 apart) -3.1%.  A slice of a wide B spans 64 rows of 32+ KB each; the
// prefetch one slice ahead brings its lines (and translations) in before
// the loads of that slice wait for them.
constexpr int64_t kPrefetchBMinStride = 16384;
constexpr int kPrefetchBMinSlices = 128;

// Byte extent [lo, hi) touched by a 2-D strided view of `rows` x `cols` elements.
struct Span {
  uintptr_t lo, hi;
};
Span span_of(const void* p, int64_t rows, int64_t cols, int64_t sr, int64_t sc, int64_t esize) {
  const uintptr_t b = (uintptr_t)p;
  const int64_t last = (rows - 1) * sr + (cols - 1) * sc;
  return {b, b + (uintptr_t)((last + 1) * esize)};
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// One operand as the kernel sees it.
struct OperandPlan {
  bool kmajor;      // K-contiguous as the kernel reads it (the original layout, or the packed copy's)
  bool pack;        // copied into the workspace (layout below)
  bool pack_mn;     // the packed copy is [K][ldp] (rows contiguous), else [rows][ldp] (K contiguous)
  int64_t ldp;      // row stride of the packed copy: its row length rounded up to 64 elements, so
                    // that every packed row starts on a 128-byte line
  int64_t ld;       // leading dimension of the direct view
  int64_t s_r, s_k; // original strides (rows = M or N)
  size_t ws_off;    // workspace offset of the packed copy
};

}  // namespace

struct gemm_plan {
  gemm_desc d;
  int device;
  int cus;
  int kind;
  int layout;
  OperandPlan a, b;
  int64_t Kp;       // K rounded up to a multiple of 8
  int splits;
  int epi;          // fused-epilogue instantiation (0: none, or the split-K reduce applies it)
  int kiters, kps;
  int tiles_m, tiles_n, total, grid, group_m;
  int round_sync;   // hand-ordered kind: round barrier per XCD (counters in the workspace)
  int b_prefetch;   // hand-ordered kind: L2 prefetch of B's slice after the next
  int tail_tiles, tail_splits, tail_kps, tail_first;  // hand-ordered kind: K-split last round
  size_t ws_partial_off;
  size_t ws_sync_off;
  size_t ws_tail_off;
  size_t ws_bytes;
};

namespace {

// Decide how an operand with logical extent rows x K and strides (s_r, s_k) is
// fed.  A packed copy is K-major [rows][ldp], or with prefer_mn rows-contiguous
// [K][ldp]: B is packed that way (unless given K-contiguous beside a
// K-contiguous A), because the producer/consumer 128x256 and 256x256 tiles
// load an N-contiguous B faster (64 k-rows of whole lines per slice instead
// of 256 rows) and the 256x128 tile is indifferent to it.
ll_status plan_operand(const char* name, int64_t rows, int64_t K, int64_t s_r, int64_t s_k, bool force_pack,
                       bool prefer_mn, OperandPlan* op) {
  op->s_r = s_r;
  op->s_k = s_k;
  if (s_k == 1) {
    op->kmajor = true;
    op->ld = s_r;
  } else if (s_r == 1) {
    op->kmajor = false;
    op->ld = s_k;
  } else {
    return fail(LL_ERR_UNSUPPORTED, "%s: neither stride is 1 (strides %lld, %lld)", name, (long long)s_r,
                (long long)s_k);
  }
  // One slice of a tile spans at most 256 rows (K-contiguous) or kBK k-rows
  // (rows contiguous) of the operand.  Keeping that span below 2^30 bytes keeps
  // every offset the loads form (a slice base below 2^30, re-based beyond it,
  // plus the span) below the descriptor's num_records clamp, so in-range data
  // is never read as out of range.
  bool direct = !force_pack && op->ld % 8 == 0;
  if (op->kmajor)
    direct = direct && K % 8 == 0 && op->ld * 2 * 256 < (1ll << 30);
  else
    direct = direct && rows % 8 == 0 && op->ld * 2 * kBK < (1ll << 30);
  op->pack = !direct;
  op->pack_mn = op->pack && prefer_mn && round_up(rows, 64) * 2 * kBK < (1ll << 30);
  op->ldp = round_up(op->pack_mn ? rows : K, 64);
  if (op->pack) op->kmajor = !op->pack_mn;
  return LL_OK;
}

int occupancy_for(int kind) {
  const KindInfo& k = kind_info(kind);
  int occ = (160 * 1024) / k.lds;
  const int waves = k.threads / 64;
  const int by_waves = 32 / waves;  // 8 waves per SIMD x 4 SIMDs upper bound
  if (occ > by_waves) occ = by_waves;
  return occ < 1 ? 1 : occ;
}

void fill_operand_args(OperandArgs* oa, const void* ptr, const OperandPlan& op, int64_t rows, int64_t K,
                       int64_t Kp, const void* ws) {
  if (op.pack && op.pack_mn) {
    oa->ptr = (const uint16_t*)((const char*)ws + op.ws_off);
    oa->ld = op.ldp;
    oa->kvalid = (int32_t)K;
    oa->extent = K * op.ldp;
  } else if (op.pack) {
    oa->ptr = (const uint16_t*)((const char*)ws + op.ws_off);
    oa->ld = op.ldp;
    oa->kvalid = (int32_t)Kp;
    oa->extent = rows * op.ldp;
  } else {
    oa->ptr = (const uint16_t*)ptr;
    oa->ld = op.ld;
    oa->kvalid = (int32_t)K;
    oa->extent = op.kmajor ? (rows - 1) * op.ld + K : (K - 1) * op.ld + rows;
  }
  oa->rows = (int32_t)rows;
}

}  // namespace

extern "C" {

const char* ll_status_string(ll_status s) {
  switch (s) {
    case LL_OK: return "LL_OK";
    case LL_ERR_INVALID_ARG: return "LL_ERR_INVALID_ARG";
    case LL_ERR_UNSUPPORTED: return "LL_ERR_UNSUPPORTED";
    case LL_ERR_WORKSPACE: return "LL_ERR_WORKSPACE";
    case LL_ERR_HIP: return "LL_ERR_HIP";
    case LL_ERR_NO_DEVICE: return "LL_ERR_NO_DEVICE";
  }
  return "LL_ERR_UNKNOWN";
}

const char* ll_last_error(void) { return g_last_error.c_str(); }

ll_status gemm_plan_create(gemm_plan** out, const gemm_desc* d) {
  if (!out || !d) return fail(LL_ERR_INVALID_ARG, "gemm_plan_create: null argument");
  *out = nullptr;
  if (d->M < 0 || d->N < 0 || d->K < 0) return fail(LL_ERR_INVALID_ARG, "negative size");
  if (d->stride_am < 1 || d->stride_ak < 1 || d->stride_bk < 1 || d->stride_bn < 1 || d->stride_cm < 1 ||
      d->stride_cn < 1)
    return fail(LL_ERR_INVALID_ARG, "strides must be >= 1");
  const uint32_t known = LL_FLAG_PACK_A | LL_FLAG_PACK_B | LL_FLAG_PRODUCER_CONSUMER | LL_FLAG_COOPERATIVE;
  if (d->flags & ~known) return fail(LL_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags & ~known);
  const uint32_t act = d->epilogue & LL_EPI_ACT_MASK;
  if ((d->epilogue & ~(LL_EPI_BIAS | LL_EPI_ACT_MASK)) || act > LL_EPI_SILU)
    return fail(LL_ERR_INVALID_ARG, "unknown epilogue 0x%x", d->epilogue);
  if ((d->flags & LL_FLAG_PRODUCER_CONSUMER) && (d->flags & LL_FLAG_COOPERATIVE))
    return fail(LL_ERR_INVALID_ARG, "LL_FLAG_PRODUCER_CONSUMER and LL_FLAG_COOPERATIVE are exclusive");
  if ((d->a_type != LL_BF16 && d->a_type != LL_F16) || d->b_type != d->a_type)
    return fail(LL_ERR_UNSUPPORTED, "A and B must both be LL_BF16 or both LL_F16");
  if (d->c_type != LL_BF16 && d->c_type != LL_F16 && d->c_type != LL_F32)
    return fail(LL_ERR_UNSUPPORTED, "C must be LL_BF16, LL_F16 or LL_F32");
  if (d->M >= (1ll << 31) || d->N >= (1ll << 31) || d->K >= (1ll << 31))
    return fail(LL_ERR_UNSUPPORTED, "dimensions must be below 2^31");

  gemm_plan p;
  memset(&p, 0, sizeof p);
  p.d = *d;
  ll_status s = plan_operand("A", d->M, d->K, d->stride_am, d->stride_ak, d->flags & LL_FLAG_PACK_A, false, &p.a);
  if (s != LL_OK) return s;
  // A packed B is N-contiguous (above), except a B given K-contiguous beside a
  // K-contiguous A: its copy stays K-contiguous (a plain copy, not a
  // transpose) for the hand-ordered kind's variant for such a B (8191 x 5003
  // x 4099, column-major B with rows 4099 elements apart: 336 -> 329 us).
  const bool b_prefer_mn = !(d->stride_bk == 1 && p.a.kmajor);
  s = plan_operand("B", d->N, d->K, d->stride_bn, d->stride_bk, d->flags & LL_FLAG_PACK_B, b_prefer_mn, &p.b);
  if (s != LL_OK) return s;
  // Any K-contiguous operand needs K padded to a multiple of 8; packed copies carry zeros there.
  p.Kp = round_up(d->K, 8);
  if (round_up(d->K, 64) * 2 * 256 >= (1ll << 30)) return fail(LL_ERR_UNSUPPORTED, "K too large");
  p.layout = layout_index(p.a.kmajor, p.b.kmajor);

  const DeviceInfo* info = nullptr;
  s = current_device(&p.device, &info);
  if (s != LL_OK) return s;
  p.cus = info->cus;

  // Tile shape: skinny M uses 128x256 tiles; tiny problems use 128x128
  // tiles; everything else tiles with separate loading waves, 128x256 when M
  // exceeds N and 256x128 otherwise (measured on the 4096^3 and the FFN
  // up/down shapes: the tile's 256-long side along the shorter of M and N
  // was 5-10% faster).
  const int64_t M = d->M, N = d->N;
  int kind;
  if (M <= 128 && N >= 1024)
    kind = KIND_TALL_PC;
  else if (M * N <= 1024ll * 1024)
    kind = KIND_SMALL_COOP;
  else
    kind = M > N ? KIND_TALL_PC : KIND_WIDE_PC;
  // Tile-count quantisation: a persistent grid runs ceil(tiles / CUs) passes
  // of tiles, so on mid-size problems a larger tile that covers the problem
  // in fewer passes wins despite more work per tile (4000x3000: 252 tiles of
  // 192x256 in one pass against 384 of 128x256 in two).  The 192x256 kind
  // (K-contiguous A only) replaces the 256x128 / 128x256 kinds when its
  // passes times tile area is at least 3% smaller and neither would split K.
  auto passes = [&](int k) -> int64_t {
    const KindInfo& ki = kind_info(k);
    const int64_t t = ((M + ki.bm - 1) / ki.bm) * ((N + ki.bn - 1) / ki.bn);
    return t * 2 <= p.cus ? -1 : (t + p.cus - 1) / p.cus;  // -1: the plan would split K
  };
  const bool free_choice = !(d->flags & (LL_FLAG_COOPERATIVE | LL_FLAG_PRODUCER_CONSUMER));
  // The hand-ordered kind moves its buffer descriptors along k and shrinks
  // their num_records with them, which is exact only while each operand, as
  // the kernel reads it, spans less than 2 GB from its base.
  auto span_bytes = [&](const OperandPlan& op, int64_t rows) -> int64_t {
    if (op.pack) return (op.pack_mn ? d->K : rows) * op.ldp * 2;
    return (op.kmajor ? (rows - 1) * op.ld + d->K : (d->K - 1) * op.ld + rows) * 2;
  };
  // The hand-ordered kind loads whole 64-deep slices with no k mask.  With K
  // not a multiple of 64 that is still exact when every operand reads zeros
  // past K: a packed copy (zero columns up to ldp, K rounded up to 64), or an
  // M/N-contiguous operand, whose k-rows past K lie beyond its descriptor
  // range.  A K-contiguous operand read in place would give its next row's
  // values there, and an Inf or NaN among them would reach C.
  const bool sq4_k_ok = d->K % 64 == 0 || ((!p.a.kmajor || p.a.pack) && (!p.b.kmajor || p.b.pack));
  const bool sq4_fits = sq4_k_ok && span_bytes(p.a, M) < 0x7FFFFFF0ll && span_bytes(p.b, N) < 0x7FFFFFF0ll;
  if (free_choice && p.a.kmajor && (kind == KIND_WIDE_PC || kind == KIND_TALL_PC)) {
    const int64_t pb = passes(kind), pt = passes(KIND_T192_PC);
    const KindInfo& kb = kind_info(kind);
    const KindInfo& kt = kind_info(KIND_T192_PC);
    if (pb > 0 && pt > 0 && pt * kt.bm * kt.bn * 100 < pb * kb.bm * kb.bn * 97) kind = KIND_T192_PC;
  }
  // Square 256x256 tiles with 8 computing waves, one per SIMD also loading
  // (KIND_SQ8_LW4), in place of 256x128: a third fewer bytes per flop through
  // each CU's load path, and one tile per CU instead of two at 4096^2.  With
  // A K-contiguous and B N-contiguous it was ahead of the 256x128 kind on
  // most shapes measured where that kind is chosen (FFN-up by 2-6%, 8192^3 by
  // up to 1%; 4096^3 within 2% either way; 4096^2 x 16384 2% behind) and behind
  // 128x256 on tall shapes (FFN-down by 7%), so it replaces only the 256x128
  // choice, only without a fused epilogue, and only when its passes times tile
  // area is no larger (it would leave CUs idle otherwise).
  if (free_choice && kind == KIND_WIDE_PC && !d->epilogue && p.a.kmajor && !p.b.kmajor) {
    const int64_t pw = passes(KIND_WIDE_PC), ps = passes(KIND_SQ8_LW4);
    const KindInfo& kw = kind_info(KIND_WIDE_PC);
    const KindInfo& ks = kind_info(KIND_SQ8_LW4);
    if (pw > 0 && ps > 0 && ps * ks.bm * ks.bn <= pw * kw.bm * kw.bn) kind = KIND_SQ8_LW4;
  }
  // Long K: beyond K = 8192 the 128x256 kind was ahead of the 256x256 and the
  // 256x128 kinds on square and wide shapes too, not only on tall ones
  // (8192^2 x 12288 .. 28672 by 4-7.5%, 8192 x 16384 x 28672 by 4%, 4096^2 x
  // 16384 by 3%; 8192^2 x 16384 1% behind), while at K <= 8192 it is not
  // (FFN-up 4% behind the 256x256 kind).  Same layout and epilogue conditions
  // as above, and again no more passes times tile area.
  if (free_choice && !d->epilogue && p.a.kmajor && !p.b.kmajor && d->K > 8192 &&
      (kind == KIND_WIDE_PC || kind == KIND_SQ8_LW4)) {
    const int64_t pk = passes(kind), pt = passes(KIND_TALL_PC);
    const KindInfo& kk = kind_info(kind);
    const KindInfo& kt = kind_info(KIND_TALL_PC);
    if (pk > 0 && pt > 0 && pt * kt.bm * kt.bn <= pk * kk.bm * kk.bn) kind = KIND_TALL_PC;
  }
  // The hand-ordered 256x256 kind (four 128x128 waves, gemm_sq4.hpp) is
  // ahead of every kind above wherever it applies: A K-contiguous or
  // M-contiguous (C = X^T Y, a layer's weight gradient), B N-contiguous or
  // K-contiguous (C = X W^T, the usual layout of a linear layer's weight);
  // one variant per layout, the M-contiguous A tiles laid out and read like
  // an N-contiguous B's and the K-contiguous B tiles like a K-contiguous A's;
  // K a multiple of 64 or the operands reading zeros past it; with or
  // without a fused epilogue.  Per pass and tile area it runs ~1.3x as fast as the others,
  // so it takes over when its passes times tile area is at most 1.25x theirs
  // and neither choice would split K; a last round it splits along K (the
  // tail split below) counts as 1/s of a pass.  Measured against the kind
  // the area rule alone picks, same operands, before the tail split existed:
  // at 1.11x (8448^2 x 4096) +18%, 1.14x (12288 x 4608 x 8192) +16%, 1.2x
  // (8191 x 5003 x 4099, both packed) +10%; at 1.33x (4608^2 x 4096, 6144^2 x
  // 4096, 4608 x 8192 x 4096) -4 to -9%.  With it those three run +19%,
  // +3.5% and +5.5% (their last rounds split 3, 4 and 4 ways), 4608^2 x 8192
  // +33%, 4352^2 x 2048 +3.4%; 4352^2 x 1024 (too short to split) -1.3%.
  if (free_choice && sq4_fits &&
      (kind == KIND_WIDE_PC || kind == KIND_TALL_PC || kind == KIND_SQ8_LW4 || kind == KIND_T192_PC)) {
    const int64_t pc = passes(kind), ph = passes(KIND_SQ4_HO);
    const KindInfo& kc = kind_info(kind);
    if (pc > 0 && ph > 0) {
      // passes in twelfths: whole rounds, and a split last round at 1/s
      const int64_t tiles_h = ((M + 255) / 256) * ((N + 255) / 256);
      const int kiters_h = (int)((round_up(d->K, 64) + 63) / 64);
      const int s = tail_splits_for(tiles_h, p.cus, kiters_h);
      const int64_t ph12 = s > 1 ? 12 * (tiles_h / p.cus) + 12 / s : 12 * ph;
      if (ph12 * 256 * 256 * 4 <= 12 * pc * kc.bm * kc.bn * 5) kind = KIND_SQ4_HO;
    }
  }
  if (d->flags & LL_FLAG_COOPERATIVE) {
    if (kind == KIND_WIDE_PC) kind = KIND_SQ8_K64;
    else if (kind_info(kind).nprod > 0) kind = KIND_WIDE_COOP;
  } else if (d->flags & LL_FLAG_PRODUCER_CONSUMER) {
    if (kind_info(kind).nprod == 0) kind = KIND_WIDE_PC;
  }
  // LL_GEMM_KIND=<kind name or index> overrides the choice (configuration sweeps).
  if (const char* env = getenv("LL_GEMM_KIND")) {
    for (int i = 0; i < KIND_COUNT; ++i)
      if (strcmp(env, kind_info(i).name) == 0) kind = i;
    if (env[0] >= '0' && env[0] <= '9' && atoi(env) < KIND_COUNT) kind = atoi(env);
  }
  // A fused epilogue runs in the kinds instantiated with it (the
  // producer/consumer tiles of the same orientation rule).
  if (d->epilogue && !kind_info(kind).epi) {
    if (d->flags & LL_FLAG_COOPERATIVE)
      return fail(LL_ERR_UNSUPPORTED, "fused epilogues run in the producer/consumer kernels only");
    kind = M > N ? KIND_TALL_PC : KIND_WIDE_PC;
  }
  {
    // A tile whose M/N-contiguous operand rows do not divide a 1-KB load (192
    // elements) exists only for K-contiguous operands (a forced kind may ask).
    const KindInfo& kv = kind_info(kind);
    if ((!p.a.kmajor && 64 % (kv.bm / 8) != 0) || (!p.b.kmajor && 64 % (kv.bn / 8) != 0))
      return fail(LL_ERR_UNSUPPORTED, "kernel %s needs K-contiguous operands for its %dx%d tile", kv.name, kv.bm,
                  kv.bn);
    // The hand-ordered kind reads A and B either way (as given or packed) in
    // whole 64-deep slices.
    if (kind == KIND_SQ4_HO && !sq4_fits)
      return fail(LL_ERR_UNSUPPORTED,
                  "kernel %s needs K a multiple of 64 (or every K-contiguous operand packed) and operands below "
                  "2 GB",
                  kv.name);
  }
  p.kind = kind;
  const KindInfo& ki = kind_info(kind);
  p.tiles_m = (int)((M + ki.bm - 1) / ki.bm);
  p.tiles_n = (int)((N + ki.bn - 1) / ki.bn);
  p.kiters = (int)((p.Kp + ki.kt - 1) / ki.kt);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  if (tiles >= (1ll << 30)) return fail(LL_ERR_UNSUPPORTED, "too many tiles");
  const int occ = occupancy_for(kind);
  const int64_t slots = (int64_t)p.cus * occ;
  // Split K when the tiles alone cannot fill the chip and K is long enough to share.
  int splits = 1;
  if (tiles > 0 && tiles * 2 <= slots && p.Kp >= 1024) {
    int64_t want = slots / tiles;
    int64_t by_k = p.Kp / 512;
    splits = (int)(want < by_k ? want : by_k);
    if (splits < 1) splits = 1;
    if (splits > 64) splits = 64;
  }
  p.kps = (p.kiters + splits - 1) / splits;
  splits = p.kiters > 0 ? (p.kiters + p.kps - 1) / p.kps : 1;  // every split gets >= 1 k-step
  // Split-K partials are raw sums; the reduce then applies the epilogue.
  p.epi = (d->epilogue && splits == 1) ? (int)((d->epilogue & LL_EPI_ACT_MASK) >> 4) + 1 : 0;
  p.splits = splits;
  p.total = (int)(tiles * splits);
  p.grid = (int)(p.total < slots ? p.total : slots);
  if (p.grid < 1) p.grid = 1;
  p.group_m = 8;
  // Tail split for the hand-ordered kind: when the last round of a
  // persistent grid holds at most half as many tiles as there are
  // workgroups, the rest of the chip would idle through it.  Those tiles are
  // split along K instead (s ways, s * tiles <= grid), their splits write raw
  // fp32 partials to the workspace, and a reduce kernel sums them in
  // ascending order and applies the epilogue.  The round then takes about
  // 1/s of its time.  LL_GEMM_TAIL_SPLIT=0 turns it off (measurement).
  p.tail_tiles = 0;
  p.tail_splits = 1;
  p.tail_kps = p.kiters;
  p.tail_first = p.total;
  if (kind == KIND_SQ4_HO && splits == 1) {
    const int s = tail_splits_for(tiles, p.grid, p.kiters);
    if (s >= 2) {
      const int64_t last = tiles % p.grid;
      p.tail_tiles = (int)last;
      p.tail_splits = s;
      p.tail_kps = (p.kiters + s - 1) / s;
      p.tail_first = (int)(tiles - last);
      p.total = p.tail_first + (int)last * s;
    }
  }
  // Round barrier per XCD for the hand-ordered kind (gemm_sq4.hpp): on
  // FFN-up (28 rounds of 256 tiles) it cut the bytes fetched past L2 from
  // 16.9 to 12.1 GB and the time by 2-5%.  It needs the grid to be whole
  // XCDs (the work-item remap) and many long rounds (kRoundSyncMinRounds,
  // kRoundSyncMinSlices).
  // LL_GEMM_ROUND_SYNC=0 / 1 overrides the choice (measurement).
  {
    const int rounds = p.grid > 0 ? (p.total + p.grid - 1) / p.grid : 0;
    p.round_sync = kind == KIND_SQ4_HO && p.grid % 8 == 0 && rounds >= kRoundSyncMinRounds &&
                   p.kiters >= kRoundSyncMinSlices;
    if (const char* env = getenv("LL_GEMM_ROUND_SYNC"))
      p.round_sync = env[0] == '1' && kind == KIND_SQ4_HO && p.grid % 8 == 0 && rounds >= 2;
  }

  {
    // B wide: an N-contiguous B's row stride as the kernel reads it (at least
    // N), or N for a K-contiguous one.  Same box, 16384 x 28672 x 8192 with B
    // K-contiguous: +6.3%; 16384 x 8192 x 28672 and 8192^3 -2%.
    const int64_t b_width = p.b.kmajor ? d->N : (p.b.pack ? p.b.ldp : p.b.ld);
    p.b_prefetch = kind == KIND_SQ4_HO && b_width >= kPrefetchBMinStride && p.kiters >= kPrefetchBMinSlices;
    if (const char* env = getenv("LL_GEMM_PREFETCH_B")) p.b_prefetch = env[0] == '1' && kind == KIND_SQ4_HO;
  }

  size_t off = 0;
  if (p.a.pack) {
    p.a.ws_off = off;
    off = align256(off + (size_t)(M * p.a.ldp * 2));
  }
  if (p.b.pack) {
    p.b.ws_off = off;
    off = align256(off + (size_t)((p.b.pack_mn ? d->K : N) * p.b.ldp * 2));
  }
  p.ws_partial_off = off;
  if (splits > 1) off = align256(off + (size_t)splits * M * N * 4);
  p.ws_sync_off = off;
  if (p.round_sync) off = align256(off + kRoundSyncWords * 4);
  p.ws_tail_off = off;
  if (p.tail_tiles > 0) off = align256(off + (size_t)p.tail_tiles * p.tail_splits * 256 * 256 * 4);
  p.ws_bytes = off;

  gemm_plan* h = new (std::nothrow) gemm_plan(p);
  if (!h) return fail(LL_ERR_INVALID_ARG, "out of host memory");
  *out = h;
  return ok();
}

ll_status gemm_plan_workspace_size(const gemm_plan* p, size_t* bytes) {
  if (!p || !bytes) return fail(LL_ERR_INVALID_ARG, "null argument");
  *bytes = p->ws_bytes;
  return ok();
}

ll_status gemm_plan_describe(const gemm_plan* p, char* buf, size_t len) {
  if (!p || !buf || len == 0) return fail(LL_ERR_INVALID_ARG, "null argument");
  const KindInfo& k = kind_info(p->kind);
  static const char* lay[4] = {"A:K-major,B:K-major", "A:K-major,B:N-major", "A:M-major,B:K-major",
                               "A:M-major,B:N-major"};
  snprintf(buf, len,
           "kernel=%s tile=%dx%d layout=%s packA=%d packB=%d tiles=%dx%d splitk=%d kiters=%d grid=%d cus=%d "
           "group_m=%d ws=%zu epilogue=0x%x fused=%d round_sync=%d tail=%dx%d prefetch_b=%d",
           k.name, k.bm, k.bn, lay[p->layout], (int)p->a.pack, (int)p->b.pack, p->tiles_m, p->tiles_n, p->splits,
           p->kiters, p->grid, p->cus, p->group_m, p->ws_bytes, p->d.epilogue, p->epi, p->round_sync, p->tail_tiles,
           p->tail_splits, p->b_prefetch);
  return ok();
}

ll_status gemm_plan_destroy(gemm_plan* p) {
  delete p;
  return ok();
}

static ll_status gemm_run_impl(const gemm_plan* p, const void* A, const void* B, void* C, const float* bias,
                               void* ws, size_t ws_bytes, void* stream);

ll_status gemm_run_ex(const gemm_plan* p, const void* A, const void* B, void* C, const float* bias, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!p) return fail(LL_ERR_INVALID_ARG, "null plan");
  const bool has_bias = p->d.epilogue & LL_EPI_BIAS;
  if (has_bias && !bias) return fail(LL_ERR_INVALID_ARG, "the plan's epilogue adds a bias: bias is null");
  if (has_bias && ((uintptr_t)bias & 3)) return fail(LL_ERR_INVALID_ARG, "bias must be 4-byte aligned");
  return gemm_run_impl(p, A, B, C, has_bias ? bias : nullptr, ws, ws_bytes, stream);
}

ll_status gemm_run(const gemm_plan* p, const void* A, const void* B, void* C, void* ws, size_t ws_bytes,
                   void* stream) {
  if (p && (p->d.epilogue & LL_EPI_BIAS))
    return fail(LL_ERR_INVALID_ARG, "the plan's epilogue adds a bias: use gemm_run_ex");
  return gemm_run_impl(p, A, B, C, nullptr, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free GEMM: the plan's workspace (packed operand copies, split-K
// partials) lives in a file-scope device array instead of a caller buffer.
// Each device holds its own copy of the array from module load until the
// process ends; its address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current (the array's name in host code is
// a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------

}  // extern "C"

static __device__ __align__(256) unsigned char scratch[LL_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

ll_status scratch_on_device(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & 255)) return fail(LL_ERR_HIP, "scratch array address %p not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LL_OK;
}
}  // namespace

extern "C" {

ll_status gemm_run_noalloc(const gemm_plan* p, const void* A, const void* B, void* C, const float* bias,
                           void* stream) {
  if (!p) return fail(LL_ERR_INVALID_ARG, "null plan");
  if (p->ws_bytes > (size_t)LL_NOALLOC_SCRATCH_BYTES)
    return fail(LL_ERR_WORKSPACE, "plan needs %zu bytes of workspace; gemm_run_noalloc holds at most %zu",
                p->ws_bytes, (size_t)LL_NOALLOC_SCRATCH_BYTES);
  const bool has_bias = p->d.epilogue & LL_EPI_BIAS;
  if (has_bias && !bias) return fail(LL_ERR_INVALID_ARG, "the plan's epilogue adds a bias: bias is null");
  if (has_bias && ((uintptr_t)bias & 3)) return fail(LL_ERR_INVALID_ARG, "bias must be 4-byte aligned");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) return fail(LL_ERR_INVALID_ARG, "plan made for device %d, current is %d", p->device, dev);
  void* ws = nullptr;
  if (p->ws_bytes > 0) {
    const ll_status s = scratch_on_device(dev, &ws);
    if (s != LL_OK) return s;
  }
  return gemm_run_impl(p, A, B, C, has_bias ? bias : nullptr, ws, ws ? (size_t)LL_NOALLOC_SCRATCH_BYTES : 0,
                       stream);
}

static ll_status gemm_run_impl(const gemm_plan* p, const void* A, const void* B, void* C, const float* bias,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!p) return fail(LL_ERR_INVALID_ARG, "null plan");
  const gemm_desc& d = p->d;
  if (d.M == 0 || d.N == 0) return ok();
  if (!C) return fail(LL_ERR_INVALID_ARG, "null C");
  if (d.K > 0 && (!A || !B)) return fail(LL_ERR_INVALID_ARG, "null A or B");
  if (ws_bytes < p->ws_bytes || (p->ws_bytes > 0 && !ws))
    return fail(LL_ERR_WORKSPACE, "workspace %zu bytes, plan needs %zu", ws_bytes, p->ws_bytes);
  if (p->ws_bytes > 0 && ((uintptr_t)ws & 255))
    return fail(LL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) return fail(LL_ERR_INVALID_ARG, "plan made for device %d, current is %d", p->device, dev);
  const int64_t csz = d.c_type == LL_F32 ? 4 : 2;
  const Span sc = span_of(C, d.M, d.N, d.stride_cm, d.stride_cn, csz);
  if (d.K > 0) {
    if (overlaps(sc, span_of(A, d.M, d.K, d.stride_am, d.stride_ak, 2)) ||
        overlaps(sc, span_of(B, d.K, d.N, d.stride_bk, d.stride_bn, 2)))
      return fail(LL_ERR_INVALID_ARG, "C overlaps A or B");
  }
  if (p->ws_bytes > 0 && overlaps(sc, Span{(uintptr_t)ws, (uintptr_t)ws + p->ws_bytes}))
    return fail(LL_ERR_INVALID_ARG, "C overlaps the workspace");
  hipStream_t st = (hipStream_t)stream;
  const int cfmt = d.c_type == LL_BF16 ? 1 : d.c_type == LL_F16 ? 2 : 0;
  const int act = (int)((d.epilogue & LL_EPI_ACT_MASK) >> 4);  // 0 none, 1 ReLU, 2 GELU, 3 SiLU
  if (d.K == 0) {
    e = launch_fill_zero(C, d.M, d.N, d.stride_cm, d.stride_cn, cfmt, bias, act, st);
    return e == hipSuccess ? ok() : hip_fail(e, "fill_zero launch");
  }
  if ((!p->a.pack && ((uintptr_t)A & 15)) || (!p->b.pack && ((uintptr_t)B & 15)))
    return fail(LL_ERR_INVALID_ARG, "A and B must be 16-byte aligned unless packed (LL_FLAG_PACK_A/B)");
  if (p->a.pack) {
    e = launch_pack_kmajor((const uint16_t*)A, p->a.s_r, p->a.s_k, d.M, d.K,
                           (uint16_t*)((char*)ws + p->a.ws_off), p->a.ldp, st);
    if (e != hipSuccess) return hip_fail(e, "pack A launch");
  }
  if (p->b.pack) {
    uint16_t* dst = (uint16_t*)((char*)ws + p->b.ws_off);
    e = p->b.pack_mn ? launch_pack_mnmajor((const uint16_t*)B, p->b.s_r, p->b.s_k, d.N, d.K, dst, p->b.ldp, st)
                     : launch_pack_kmajor((const uint16_t*)B, p->b.s_r, p->b.s_k, d.N, d.K, dst, p->b.ldp, st);
    if (e != hipSuccess) return hip_fail(e, "pack B launch");
  }
  GemmKArgs k;
  memset(&k, 0, sizeof k);
  fill_operand_args(&k.a, A, p->a, d.M, d.K, p->Kp, ws);
  fill_operand_args(&k.b, B, p->b, d.N, d.K, p->Kp, ws);
  k.M = (int32_t)d.M;
  k.N = (int32_t)d.N;
  k.c_fmt = cfmt;
  k.bias = bias;
  k.act = act;
  k.splits = p->splits;
  k.kiters = p->kiters;
  k.kps = p->kps;
  k.tiles_m = p->tiles_m;
  k.tiles_n = p->tiles_n;
  k.group_m = p->group_m;
  k.total = p->total;
  // an operand that only one row (column) of tiles reads is loaded once
  k.a.once = p->tiles_n == 1;
  k.b.once = p->tiles_m == 1;
  if (p->splits > 1) {
    k.partial = (float*)((char*)ws + p->ws_partial_off);
  } else {
    k.c = C;
    k.ldcm = d.stride_cm;
    k.ldcn = d.stride_cn;
    k.c_fast = d.stride_cn == 1 && d.stride_cm % 2 == 0 && ((uintptr_t)C & 3) == 0 &&
               d.stride_cm * (d.M + 256) < (1ll << 31);
  }
  k.b_prefetch = p->b_prefetch;
  k.tail_first = p->tail_first;
  k.tail_splits = p->tail_splits;
  k.tail_kps = p->tail_kps;
  if (p->tail_tiles > 0) k.tail_partial = (float*)((char*)ws + p->ws_tail_off);
  if (p->round_sync) {
    k.sync = (uint32_t*)((char*)ws + p->ws_sync_off);
    e = launch_clear_words(k.sync, kRoundSyncWords, st);
    if (e != hipSuccess) return hip_fail(e, "round counter clear launch");
  }
  e = p->epi ? launch_gemm_epi(p->layout, p->kind, d.a_type == LL_F16, p->epi, k, p->grid, st)
             : launch_gemm(p->layout, p->kind, d.a_type == LL_F16, k, p->grid, st);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  if (p->tail_tiles > 0) {
    e = launch_tail_reduce(k.tail_partial, p->tail_splits, p->tail_first, p->tail_tiles, p->tiles_m, p->tiles_n,
                           p->group_m, d.M, d.N, C, d.stride_cm, d.stride_cn, cfmt, bias, act, st);
    if (e != hipSuccess) return hip_fail(e, "tail reduce launch");
  }
  if (p->splits > 1) {
    e = launch_splitk_reduce(k.partial, p->splits, d.M, d.N, C, d.stride_cm, d.stride_cn, cfmt, bias, act, st);
    if (e != hipSuccess) return hip_fail(e, "split-K reduce launch");
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Linear compression
// ---------------------------------------------------------------------------

static ll_status lincomp_check(const lincomp_desc* d, bool ragged = false) {
  if (!d) return fail(LL_ERR_INVALID_ARG, "null desc");
  if (d->R < 0 || d->C < 0 || d->Nu < 0 || d->Ni < 0 || d->D < 0 || d->Mo < 0)
    return fail(LL_ERR_INVALID_ARG, "negative size");
  if (d->flags & ~(uint32_t)LL_LINCOMP_NO_DEDUP) return fail(LL_ERR_INVALID_ARG, "unknown flag bits");
  if ((d->epilogue & ~(LL_EPI_BIAS | LL_EPI_ACT_MASK)) || (d->epilogue & LL_EPI_ACT_MASK) > LL_EPI_SILU)
    return fail(LL_ERR_INVALID_ARG, "unknown epilogue 0x%x", d->epilogue);
  if (d->y_type != LL_BF16 && d->y_type != LL_F32) return fail(LL_ERR_UNSUPPORTED, "Y must be LL_BF16 or LL_F32");
  if (d->D % 8 || d->Mo % 8) return fail(LL_ERR_INVALID_ARG, "D and Mo must be multiples of 8");
  if (d->su_n % 8 || d->si_n % 8 || d->sw_n % 8 || d->su_r % 8 || d->su_c % 8 || d->si_r % 8 || d->si_c % 8 ||
      d->sy_r % 8 || d->sy_c % 8 || d->sy_m % 8)
    return fail(LL_ERR_INVALID_ARG, "every row and batch stride must be a multiple of 8");
  if (d->su_n < d->D || d->si_n < d->D || d->sw_n < d->Mo || d->sy_m < d->D)
    return fail(LL_ERR_INVALID_ARG, "row strides shorter than the rows");
  if (d->su_r < 0 || d->su_c < 0 || d->si_r < 0 || d->si_c < 0 || d->sy_r < 0 || d->sy_c < 0)
    return fail(LL_ERR_INVALID_ARG, "negative stride");
  if (d->Mo >= (1 << 30) || d->D >= (1 << 30) || (ragged ? d->C : d->R * d->C) >= (1ll << 30) ||
      d->R >= (1ll << 30))
    return fail(LL_ERR_UNSUPPORTED, ragged ? "Mo, D, R and Ctot must be below 2^30"
                                           : "Mo, D and R*C must be below 2^30");
  if (d->su_n * 2 * kBK >= (1ll << 31) || d->si_n * 2 * kBK >= (1ll << 31) || d->sw_n * 2 * kBK >= (1ll << 31))
    return fail(LL_ERR_UNSUPPORTED, "row strides too large");
  // the kernel keeps every stride in 32 bits
  for (int64_t st : {d->su_r, d->su_c, d->su_n, d->si_r, d->si_c, d->si_n, d->sw_n, d->sy_r, d->sy_c, d->sy_m})
    if (st >= (1ll << 31)) return fail(LL_ERR_UNSUPPORTED, "strides must be below 2^31 elements");
  // one candidate's Y block is addressed with 32-bit element offsets
  if ((d->Mo + 1) * d->sy_m >= (1ll << 30)) return fail(LL_ERR_UNSUPPORTED, "Mo * sy_m too large");
  return LL_OK;
}

ll_status lincomp_workspace_size(const lincomp_desc* d, size_t* bytes) {
  ll_status s = lincomp_check(d);
  if (s != LL_OK) return s;
  if (!bytes) return fail(LL_ERR_INVALID_ARG, "null bytes");
  *bytes = 0;  // the fused kernel keeps the per-request user contribution in registers
  return ok();
}

// Shared by the per-request and the ragged entry points.  offsets != nullptr:
// ragged (d->C is the total candidate count; d's request strides of item and
// Y and the per-candidate user stride are 0).
static ll_status lincomp_launch(const lincomp_desc* d, const int64_t* offsets, const void* user, const void* item,
                                const void* W, const float* bias, void* Y, void* stream) {
  ll_status s = lincomp_check(d, offsets != nullptr);
  if (s != LL_OK) return s;
  if (d->epilogue & LL_EPI_BIAS) {
    if (!bias) return fail(LL_ERR_INVALID_ARG, "the epilogue adds a bias: bias is null");
    if ((uintptr_t)bias & 15) return fail(LL_ERR_INVALID_ARG, "bias must be 16-byte aligned");
  } else {
    bias = nullptr;
  }
  if (d->R == 0 || d->C == 0 || d->Mo == 0 || d->D == 0) return ok();
  if (!Y || !W || (d->Nu > 0 && !user) || (d->Ni > 0 && !item)) return fail(LL_ERR_INVALID_ARG, "null pointer");
  if (((uintptr_t)user & 15) || ((uintptr_t)item & 15) || ((uintptr_t)W & 15) || ((uintptr_t)Y & 15))
    return fail(LL_ERR_INVALID_ARG, "user, item, W and Y must be 16-byte aligned");
  const DeviceInfo* info = nullptr;
  int dev = 0;
  s = current_device(&dev, &info);
  if (s != LL_OK) return s;
  const int64_t ysz = d->y_type == LL_BF16 ? 2 : 4;
  const Span sy = {(uintptr_t)Y, (uintptr_t)Y + (uintptr_t)(((d->R - 1) * d->sy_r + (d->C - 1) * d->sy_c +
                                                              (d->Mo - 1) * d->sy_m + d->D) * ysz)};
  if (overlaps(sy, Span{(uintptr_t)W, (uintptr_t)W + (uintptr_t)((d->Nu + d->Ni - 1) * d->sw_n + d->Mo) * 2}) ||
      (d->Nu > 0 && overlaps(sy, Span{(uintptr_t)user, (uintptr_t)user + (uintptr_t)(((d->R - 1) * d->su_r +
                                                                                      (d->C - 1) * d->su_c +
                                                                                      (d->Nu - 1) * d->su_n + d->D) * 2)})) ||
      (d->Ni > 0 && overlaps(sy, Span{(uintptr_t)item, (uintptr_t)item + (uintptr_t)(((d->R - 1) * d->si_r +
                                                                                      (d->C - 1) * d->si_c +
                                                                                      (d->Ni - 1) * d->si_n + d->D) * 2)})))
    return fail(LL_ERR_INVALID_ARG, "Y overlaps an input");

  const LincompKind& lk = lincomp_kind();
  LincompKArgs k;
  memset(&k, 0, sizeof k);
  k.user = (const uint16_t*)user;
  k.item = (const uint16_t*)item;
  k.W = (const uint16_t*)W;
  k.Y = Y;
  k.su_r = (int32_t)d->su_r;
  k.su_c = (int32_t)d->su_c;
  k.su_n = (int32_t)d->su_n;
  k.si_r = (int32_t)d->si_r;
  k.si_c = (int32_t)d->si_c;
  k.si_n = (int32_t)d->si_n;
  k.sw_n = (int32_t)d->sw_n;
  k.sy_r = (int32_t)d->sy_r;
  k.sy_c = (int32_t)d->sy_c;
  k.sy_m = (int32_t)d->sy_m;
  k.user_extent = d->Nu > 0 ? (d->R - 1) * d->su_r + (d->C - 1) * d->su_c + (d->Nu - 1) * d->su_n + d->D : 0;
  k.item_extent = d->Ni > 0 ? (d->R - 1) * d->si_r + (d->C - 1) * d->si_c + (d->Ni - 1) * d->si_n + d->D : 0;
  k.w_extent = (d->Nu + d->Ni - 1) * d->sw_n + d->Mo;
  k.R = (int32_t)d->R;
  k.C = (int32_t)d->C;
  k.Nu = (int32_t)d->Nu;
  k.Ni = (int32_t)d->Ni;
  k.D = (int32_t)d->D;
  k.Mo = (int32_t)d->Mo;
  k.tiles_m = (int32_t)((d->Mo + lk.bm - 1) / lk.bm);
  k.tiles_n = (int32_t)((d->D + lk.bn - 1) / lk.bn);
  k.nu_sl = (int32_t)((d->Nu + lk.kt - 1) / lk.kt);
  // A candidate with no item rows still needs one (all-zero) slice so that its
  // result (the user contribution alone) is written.
  k.ni_sl = d->Ni > 0 ? (int32_t)((d->Ni + lk.kt - 1) / lk.kt) : 1;
  const int64_t tiles = (int64_t)k.tiles_m * k.tiles_n;
  int64_t total;
  if (offsets) {
    // Equal contiguous ranges of the flat candidate axis, one per CU and
    // output tile: the work is balanced whatever the request lengths; a range
    // recomputes the user block of each request it touches (at most one more
    // than the requests it holds whole).
    k.offsets = offsets;
    k.nranges = (int32_t)std::max<int64_t>(1, std::min<int64_t>(d->C, info->cus / std::max<int64_t>(1, tiles)));
    k.chunk = 1;
    k.nchunks = 1;
    total = tiles * k.nranges;
  } else {
    // Candidates per work item: one workgroup per CU, and the user block is
    // recomputed only once per work item.
    const int64_t per_req = std::max<int64_t>(1, (info->cus + d->R * tiles - 1) / (d->R * tiles));
    int64_t chunk = (d->C + per_req - 1) / per_req;
    if (chunk < 1) chunk = 1;
    k.chunk = (int32_t)chunk;
    k.nchunks = (int32_t)((d->C + chunk - 1) / chunk);
    total = tiles * d->R * k.nchunks;
  }
  if (total >= (1ll << 30)) return fail(LL_ERR_UNSUPPORTED, "too many work items");
  k.total = (int32_t)total;
  k.y_bf16 = d->y_type == LL_BF16;
  // Y and its strides are 16-byte multiples (checked above): bf16 Y tiles
  // that lie wholly inside Y leave through LDS in whole lines
  k.y_stage = k.y_bf16;
  // Per-candidate user rows (su_c != 0) leave nothing to share.
  k.dedup = !(d->flags & LL_LINCOMP_NO_DEDUP) && d->su_c == 0;
  k.bias = bias;
  const int grid = (int)std::min<int64_t>(total, info->cus);
  hipError_t e = launch_lincomp(k, (int)((d->epilogue & LL_EPI_ACT_MASK) >> 4), grid, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lincomp launch");
  return ok();
}

ll_status lincomp_run(const lincomp_desc* d, const void* user, const void* item, const void* W, void* Y,
                      void* ws, size_t ws_bytes, void* stream) {
  if (d && (d->epilogue & LL_EPI_BIAS))
    return fail(LL_ERR_INVALID_ARG, "the epilogue adds a bias: use lincomp_run_ex");
  return lincomp_run_ex(d, user, item, W, nullptr, Y, ws, ws_bytes, stream);
}

ll_status lincomp_run_ex(const lincomp_desc* d, const void* user, const void* item, const void* W,
                         const float* bias, void* Y, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  return lincomp_launch(d, nullptr, user, item, W, bias, Y, stream);
}

ll_status lincomp_ragged_run(const lincomp_ragged_desc* g, const int64_t* offsets, const void* user,
                             const void* item, const void* W, void* Y, void* stream) {
  if (g && (g->epilogue & LL_EPI_BIAS))
    return fail(LL_ERR_INVALID_ARG, "the epilogue adds a bias: use lincomp_ragged_run_ex");
  return lincomp_ragged_run_ex(g, offsets, user, item, W, nullptr, Y, stream);
}

ll_status lincomp_ragged_run_ex(const lincomp_ragged_desc* g, const int64_t* offsets, const void* user,
                                const void* item, const void* W, const float* bias, void* Y, void* stream) {
  if (!g) return fail(LL_ERR_INVALID_ARG, "null desc");
  lincomp_desc d;
  memset(&d, 0, sizeof d);
  d.R = g->R;
  d.C = g->Ctot;
  d.Nu = g->Nu;
  d.Ni = g->Ni;
  d.D = g->D;
  d.Mo = g->Mo;
  d.su_r = g->su_r;
  d.su_n = g->su_n;
  d.si_c = g->si_c;
  d.si_n = g->si_n;
  d.sw_n = g->sw_n;
  d.sy_c = g->sy_c;
  d.sy_m = g->sy_m;
  d.y_type = g->y_type;
  d.flags = g->flags;
  d.epilogue = g->epilogue;
  if (!offsets && g->R > 0 && g->Ctot > 0) {
    ll_status s = lincomp_check(&d, true);
    return s != LL_OK ? s : fail(LL_ERR_INVALID_ARG, "null offsets");
  }
  return lincomp_launch(&d, offsets ? offsets : (const int64_t*)nullptr, user, item, W, bias, Y, stream);
}

}  // extern "C"
