/*
 * linlayers.h -- C ABI of the MI355X (gfx950) GEMM and RecSys linear-compression
 * library (liblinlayers.so).
 *
 * Operations (definitions from the pages this library follows):
 *
 *  - gemm_*   : C = act(A.B + bias) with bf16 (or fp16) A and B, fp32
 *               accumulation, fp32, bf16 or fp16 C; bias and activation optional.
 *               The problem is stated as on the page "Triton 3.7 permite
 *               extender el compilador de GPU sin forks" (listings in the
 *               sections "NVIDIA H100 (Hopper): GEMM persistente" and
 *               "AMD MI350: GEMM segmentado"): pointers a/b/c, sizes M, N, K and
 *               the element strides stride_am, stride_ak, stride_bk, stride_bn,
 *               stride_cm, stride_cn.  The tile sizes and stage count those
 *               listings take as compile-time constants are chosen inside the
 *               plan here.
 *  - lincomp_*: the RecSys linear-compression layer named on the page "Meta
 *               accelere un noyau GPU d'un facteur 4 avec TLX" (section on what
 *               a four-fold speed-up means).  For request r and candidate c the
 *               layer input X is the request's user rows stacked above the
 *               candidate's item rows, and Y[r][c] = W^T . X.  The user rows are
 *               identical across a request's candidates (section on how data
 *               loading holds back compute), so this entry point takes them
 *               once per request and computes their contribution once per
 *               request, not once per candidate.
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers named A, B, C, user, item, W, Y and workspace are DEVICE
 *    pointers on the device the plan (or call) runs on; descriptors and plans
 *    are host memory.  The caller owns every buffer, including the workspace;
 *    the library never allocates device memory.  It owns only host plan
 *    objects (released by gemm_plan_destroy).
 *  - bf16 values are passed as their 16-bit patterns.  All strides are in
 *    ELEMENTS, not bytes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Run calls only
 *    enqueue work and return; results are ready when the stream is.  Errors
 *    raised by the device (faults) surface at the caller's next
 *    synchronisation, not as a return value.
 *  - No exceptions cross this ABI.  Every call returns an ll_status.
 *  - Plans are immutable and may be shared between host threads; concurrent
 *    runs need distinct workspaces.
 */
#ifndef LINLAYERS_H
#define LINLAYERS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LL_OK = 0,
  LL_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad stride, overlap, wrong device */
  LL_ERR_UNSUPPORTED = 2,  /* dtype, layout or device (not gfx950) this library does not handle */
  LL_ERR_WORKSPACE = 3,    /* workspace smaller than the queried size */
  LL_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  LL_ERR_NO_DEVICE = 5     /* no HIP device is visible */
} ll_status;

typedef enum { LL_BF16 = 0, LL_F32 = 1, LL_F16 = 2 /* IEEE binary16 */ } ll_dtype;

/* gemm_desc.flags */
#define LL_FLAG_PACK_A 0x1u /* always copy A into an aligned workspace layout first */
#define LL_FLAG_PACK_B 0x2u /* same for B */
#define LL_FLAG_PRODUCER_CONSUMER 0x4u /* force the wave-specialised (producer/consumer) kernel */
#define LL_FLAG_COOPERATIVE 0x8u       /* force the kernel in which every wave loads and computes */

/*
 * GEMM problem.  A[i][k] = A[i*stride_am + k*stride_ak] (0 <= i < M, 0 <= k < K),
 * B[k][j] = B[k*stride_bk + j*stride_bn], C[i][j] = C[i*stride_cm + j*stride_cn].
 * a_type and b_type: both LL_BF16 or both LL_F16 (the fp16 GEMMs of the
 * tables on "Triton 3.7 permite extender el compilador de GPU sin forks");
 * c_type is LL_BF16, LL_F16 or LL_F32.  Products are accumulated in fp32.
 * For A and for B, one of the two strides must be 1 (row- or column-major, any
 * leading dimension); C may use any positive strides.  16-bit C is rounded
 * to nearest even (fp16 overflow gives infinity).
 */
/*
 * gemm_desc.epilogue: what happens to each fp32 sum z = (A.B)[i][j] before it
 * is converted to c_type (page "Meta accélère un noyau GPU d'un facteur 4 avec
 * TLX", section "Par où commencer dans votre équipe": fuse steps, then
 * measure again).  LL_EPI_BIAS adds bias[j] (fp32, one per column of C,
 * passed to gemm_run_ex); then the activation, evaluated in fp32:
 *   LL_EPI_RELU  max(z, 0)
 *   LL_EPI_GELU  z * Phi(z) = z/2 * (1 + erf(z / sqrt(2)))  (the exact form)
 *   LL_EPI_SILU  z / (1 + exp(-z))
 * 0: C = A.B as before.  Unknown bits -> LL_ERR_INVALID_ARG.
 */
#define LL_EPI_BIAS 0x1u
#define LL_EPI_RELU 0x10u
#define LL_EPI_GELU 0x20u
#define LL_EPI_SILU 0x30u
#define LL_EPI_ACT_MASK 0xF0u

typedef struct {
  int64_t M, N, K;
  int64_t stride_am, stride_ak, stride_bk, stride_bn, stride_cm, stride_cn;
  int32_t a_type, b_type, c_type; /* ll_dtype values */
  uint32_t flags;                 /* LL_FLAG_* ; unknown bits -> LL_ERR_INVALID_ARG */
  uint32_t epilogue;              /* LL_EPI_* ; 0 for a plain product */
} gemm_desc;

typedef struct gemm_plan gemm_plan; /* opaque, host-side, immutable */

/*
 * Validate `desc` and choose the kernel configuration (tile shape, stage
 * count, wave roles, split-K factor, grid) for the CURRENT HIP device.
 * On success *out receives a new plan.
 * Tile choice: 256x128 or 128x256 tiles with separate loading waves (the
 * 256-long side along the shorter of M and N); 128x256 for M <= 128; 128x128
 * for M*N <= 2^20.  The persistent grid runs ceil(tiles / CUs) passes of
 * tiles, so when A is K-contiguous (or packed) and 192x256 tiles cover the
 * problem in passes x tile area at least 3% smaller, without a K split,
 * those are used instead.  Where 256x128 remains, A is K-contiguous, B is
 * N-contiguous and no epilogue is fused, 256x256 tiles (eight computing
 * waves, one per SIMD also loading) replace it when they need no more passes
 * x tile area; for K > 8192 the 128x256 tiles take their place again under
 * the same conditions.  Last, with A K- or M-contiguous (C = X^T Y, a
 * weight gradient) and B N- or K-contiguous (C = X W^T with W stored
 * [N][K]), direct or packed, K a multiple of 64 (or every K-contiguous
 * operand packed) and each operand spanning under 2 GB from its base, any
 * of those four kinds gives way to KIND_SQ4_HO (256x256 tiles,
 * four waves of 128x128, one per SIMD, each loading and computing in one
 * hand-ordered instruction stream) when that needs at most 1.25x their
 * passes x tile area (it runs ~1.3x as fast per pass and area); with or
 * without a fused epilogue.  K is split when the tiles fill
 * fewer than half of the CUs.  KIND_SQ4_HO plans with 8 rounds or more
 * (passes of the grid over the tiles) of K >= 8192 each, on a grid of whole
 * XCDs, also keep each
 * XCD's workgroups within a round of one another (round_sync=1 in the
 * description; LL_GEMM_ROUND_SYNC=0, or 1 for two rounds or more, overrides): a bounded wait between
 * rounds, so that tiles sharing A and B panels read them from L2 together;
 * its counters take 1 KB of workspace.  When a KIND_SQ4_HO plan's last round
 * would hold at most half as many tiles as the grid has workgroups (and K
 * has at least 32 slices of 64), those tiles are split 2-4 ways along K
 * (tail=<tiles>x<splits> in the description; LL_GEMM_TAIL_SPLIT=0 turns it
 * off): each split leaves a 256x256 fp32 partial in the workspace, and a
 * reduce kernel adds them in ascending split order, then applies the
 * epilogue.  KIND_SQ4_HO plans whose B is wide (an N-contiguous B's rows, as
 * read, 16384 elements or more apart; a K-contiguous B with N >= 16384), with
 * K >= 8192, also prefetch each B slice into L2 one slice ahead (prefetch_b=1; LL_GEMM_PREFETCH_B=0 or 1 overrides).  The environment variable LL_GEMM_KIND (a
 * kernel name as printed by gemm_plan_describe, or its index) forces a
 * kernel for configuration sweeps; a forced kernel that cannot take the
 * operands (a 192-row tile with an M-contiguous A, KIND_SQ4_HO outside the
 * conditions above) gives LL_ERR_UNSUPPORTED.
 * Errors: LL_ERR_INVALID_ARG (null out/desc, negative size, zero or negative
 * stride, unknown flag bits), LL_ERR_UNSUPPORTED (dtype, neither stride of A
 * or of B equal to 1, device not gfx950), LL_ERR_NO_DEVICE, LL_ERR_HIP.
 * Argument checks run before any device query.
 */
ll_status gemm_plan_create(gemm_plan** out, const gemm_desc* desc);

/* Bytes of device workspace gemm_run needs for this plan (may be 0). */
ll_status gemm_plan_workspace_size(const gemm_plan* plan, size_t* bytes);

/*
 * Writes a one-line, NUL-terminated description of the plan's choices
 * (kernel, tile, stages, roles, split-K, grid) into buf[0..len).
 */
ll_status gemm_plan_describe(const gemm_plan* plan, char* buf, size_t len);

/*
 * C = A.B on `stream`.  A, B: device buffers of a_type (bf16 or fp16); C:
 * device buffer of c_type.  Unless the plan packs an operand (LL_FLAG_PACK_*, or a layout that
 * needs it: leading dimension not a multiple of 8, K-contiguous operand with
 * K not a multiple of 8, M- or N-contiguous operand whose M or N is not a
 * multiple of 8), that operand's pointer must be 16-byte aligned.
 * M == 0 or N == 0: nothing is written.  K == 0: C is set to zero.
 * Errors: LL_ERR_INVALID_ARG (null plan/pointer with a non-empty problem,
 * misaligned operand, C overlapping A or B, current device differs from the
 * plan's), LL_ERR_WORKSPACE (ws_bytes below gemm_plan_workspace_size, a
 * null workspace with a non-zero requirement, or a workspace not 256-byte
 * aligned), LL_ERR_HIP (launch failure).  Packed copies live in the
 * workspace with rows padded to whole 128-byte lines: A K-contiguous
 * [M][ldp], B N-contiguous [K][ldp] (K-contiguous [N][ldp] when B is given
 * K-contiguous and A is K-contiguous); so do split-K partials, the round
 * counters of plans with round_sync=1 (zeroed by the call itself) and the
 * partial tiles of a K-split last round.
 * The call only launches kernels on `stream` (pack, counter clear, GEMM,
 * split-K or tail reduce, or the K == 0 fill): it allocates nothing and records no memset or copy, so
 * it may be captured into a HIP graph; replays reuse the captured pointers.
 */
ll_status gemm_run(const gemm_plan* plan, const void* A, const void* B, void* C,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * gemm_run for a plan whose epilogue adds a bias: `bias` is a device array of
 * N fp32 values (4-byte aligned), read once per output tile.  A plan without
 * LL_EPI_BIAS ignores `bias`; gemm_run on a plan with LL_EPI_BIAS, or a null
 * bias here, is LL_ERR_INVALID_ARG.  Otherwise as gemm_run.
 */
ll_status gemm_run_ex(const gemm_plan* plan, const void* A, const void* B, void* C, const float* bias,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * gemm_run_ex without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The plan's workspace (packed operand copies,
 * split-K partials, round counters, tail partials) is taken from a device array inside the library, one per
 * GPU, LL_NOALLOC_SCRATCH_BYTES long, which each GPU the library runs on
 * holds from the library's load until the process ends.  The call allocates
 * and frees nothing and calls no allocating library routine; its first call
 * on a device looks up that device's array address once.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other streams, other host threads) race on it and give undefined
 * results; serialise them.  Each call writes every workspace byte it reads
 * before reading it, so nothing left by an earlier call matters.
 * bias: as for gemm_run_ex (required iff the plan's epilogue adds one,
 * ignored otherwise).  Results are identical to gemm_run_ex's.
 * Errors: LL_ERR_WORKSPACE if the plan needs more than
 * LL_NOALLOC_SCRATCH_BYTES (gemm_plan_workspace_size tells; nothing is
 * launched), otherwise as gemm_run_ex.
 */
#define LL_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB */
ll_status gemm_run_noalloc(const gemm_plan* plan, const void* A, const void* B, void* C, const float* bias,
                           void* stream);

ll_status gemm_plan_destroy(gemm_plan* plan);

/*
 * Linear compression.  Sizes: R requests, C candidates per request, Nu user
 * rows, Ni item rows, D columns (embedding width), Mo compressed rows.
 *   user[r][c][n][d] = user[r*su_r + c*su_c + n*su_n + d] (0 <= n < Nu), bf16
 *   item[r][c][n][d] = item[r*si_r + c*si_c + n*si_n + d] (0 <= n < Ni), bf16
 *   W[n][m] = W[n*sw_n + m]                               (0 <= n < Nu+Ni), bf16
 *   Y[r][c][m][d] = Y[r*sy_r + c*sy_c + m*sy_m + d], y_type LL_BF16 or LL_F32
 * Y[r][c][m][d] = sum_{n<Nu} W[n][m] user[r][c][n][d] + sum_{n<Ni} W[Nu+n][m] item[r][c][n][d],
 * accumulated in fp32.  su_c == 0: the user rows are one block per request,
 * shared by all its candidates (the request's repeated features); the first
 * sum is then computed once per request and kept in fp32 (never rounded to
 * bf16) until the final result is rounded.  su_c != 0: every candidate
 * carries its own user rows (a materialised stacked input [user; item] per
 * candidate, the layer's original form); each candidate then computes both
 * sums, in the same order, so equal rows give bit-identical results.
 * The last dimension of every tensor is contiguous; user, item and W must be
 * 16-byte aligned and every stride a non-negative multiple of 8 (su_n, si_n,
 * sw_n, sy_m at least the row length); D and Mo multiples of 8.
 * flags: 0 = user block once per request (default); LL_LINCOMP_NO_DEDUP =
 * treat the user rows as if they were repeated for every candidate (each
 * candidate recomputes the user contribution; the result is the same sum).
 */
#define LL_LINCOMP_NO_DEDUP 0x1u

/*
 * epilogue: what happens to each fp32 sum Y[r][c][m][d] before it is
 * converted to y_type, fused into the layer (page "Meta accélère un noyau GPU
 * d'un facteur 4 avec TLX", section "Par où commencer dans votre équipe":
 * fuse steps, then measure again).  The LL_EPI_* bits of gemm_desc:
 * LL_EPI_BIAS adds bias[m] (fp32, one per compressed row, Mo values, passed
 * to lincomp_run_ex / lincomp_ragged_run_ex), then the activation LL_EPI_RELU,
 * LL_EPI_GELU (z * Phi(z), the exact form) or LL_EPI_SILU, in fp32.
 * 0: Y = W^T . X as before.  Unknown bits -> LL_ERR_INVALID_ARG.
 */
typedef struct {
  int64_t R, C, Nu, Ni, D, Mo;
  int64_t su_r, su_c, su_n;
  int64_t si_r, si_c, si_n;
  int64_t sw_n;
  int64_t sy_r, sy_c, sy_m;
  int32_t y_type; /* ll_dtype */
  uint32_t flags;
  uint32_t epilogue; /* LL_EPI_* ; 0 for the plain layer */
} lincomp_desc;

/* Bytes of device workspace lincomp_run needs for `desc` (may be 0).
 * Errors as for the argument checks of lincomp_run; no device is queried. */
ll_status lincomp_workspace_size(const lincomp_desc* desc, size_t* bytes);

/*
 * Y = linear compression of (user, item) by W, on `stream` (current device,
 * must be gfx950).  R == 0 or C == 0: nothing is written.
 * Errors: LL_ERR_INVALID_ARG (null desc/pointer, negative size, stride or
 * alignment rule above broken, Y overlapping an input), LL_ERR_UNSUPPORTED
 * (y_type, device), LL_ERR_WORKSPACE, LL_ERR_NO_DEVICE, LL_ERR_HIP.
 * The call launches one kernel on `stream` and allocates nothing, so it may
 * be captured into a HIP graph.
 */
ll_status lincomp_run(const lincomp_desc* desc, const void* user, const void* item,
                      const void* W, void* Y, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * lincomp_run for a descriptor whose epilogue adds a bias: `bias` is a device
 * array of Mo fp32 values, 16-byte aligned, bias[m] added to every Y[.][.][m][.].
 * A descriptor without LL_EPI_BIAS ignores `bias`; lincomp_run on a descriptor
 * with LL_EPI_BIAS, or a null or misaligned bias here, is LL_ERR_INVALID_ARG.
 * Otherwise as lincomp_run.
 */
ll_status lincomp_run_ex(const lincomp_desc* desc, const void* user, const void* item, const void* W,
                         const float* bias, void* Y, void* workspace, size_t ws_bytes, void* stream);

/*
 * Linear compression over ragged requests (page "Meta accélère un noyau GPU
 * d'un facteur 4 avec TLX", sections "Comment le chargement des données gêne
 * le calcul" and "Par où commencer dans votre équipe": the number of
 * candidates scored per request varies).  Request r owns the candidates
 * offsets[r] .. offsets[r+1]-1 of a flat candidate axis of length Ctot:
 *   user[r][n][d] = user[r*su_r + n*su_n + d]   (0 <= n < Nu), bf16
 *   item[g][n][d] = item[g*si_c + n*si_n + d]   (0 <= g < Ctot, 0 <= n < Ni), bf16
 *   W as for lincomp_run; Y[g][m][d] = Y[g*sy_c + m*sy_m + d], y_type
 * Y[g] = sum_{n<Nu} W[n][m] user[r(g)][n][d] + sum_{n<Ni} W[Nu+n][m] item[g][n][d],
 * with the user sum formed once per (request, work item) and kept in fp32.
 * offsets: device array of R+1 int64, non-decreasing, offsets[0] = 0,
 * offsets[R] = Ctot (read on the device; values outside [0, Ctot] are
 * clamped, and malformed offsets give unspecified rows of Y but no access
 * outside the buffers).  Candidates of empty requests do not exist; every
 * g in [0, Ctot) is written.  Alignment and stride rules as for
 * lincomp_run.  No workspace.  R == 0 or Ctot == 0: nothing is written.
 * Errors as for lincomp_run, plus LL_ERR_INVALID_ARG for a null offsets.
 */
typedef struct {
  int64_t R, Ctot, Nu, Ni, D, Mo;
  int64_t su_r, su_n;
  int64_t si_c, si_n;
  int64_t sw_n;
  int64_t sy_c, sy_m;
  int32_t y_type; /* ll_dtype */
  uint32_t flags; /* LL_LINCOMP_NO_DEDUP or 0 */
  uint32_t epilogue; /* LL_EPI_* as for lincomp_desc */
} lincomp_ragged_desc;

ll_status lincomp_ragged_run(const lincomp_ragged_desc* desc, const int64_t* offsets, const void* user,
                             const void* item, const void* W, void* Y, void* stream);

/* lincomp_ragged_run with the bias of an LL_EPI_BIAS epilogue (as lincomp_run_ex). */
ll_status lincomp_ragged_run_ex(const lincomp_ragged_desc* desc, const int64_t* offsets, const void* user,
                                const void* item, const void* W, const float* bias, void* Y, void* stream);

/* Static, human-readable name of a status code ("LL_OK", ...). */
const char* ll_status_string(ll_status s);

/* Message of the most recent failing call on this host thread ("" if none). */
const char* ll_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LINLAYERS_H */
