/*
 * llprobes.h -- C ABI of libllprobes.so: measurement probes that find the
 * practical ceilings of the two resources the kernels of liblinlayers.so are
 * bound by, on the GPU they run on.  They compute nothing of the library's
 * operations; a benchmark times them beside the library's kernels so that a
 * kernel's fraction of the published peak can be read against what the chip
 * sustains in practice.
 *
 *  - MFMA issue: waves that do nothing but back-to-back bf16 matrix
 *    multiply-accumulates (v_mfma_f32_32x32x16_bf16, the instruction of the
 *    library's producer/consumer GEMM kinds and linear compression, or
 *    v_mfma_f32_16x16x32_bf16, that of its hand-ordered GEMM kind), with no
 *    memory traffic and no dependency stalls.  Its rate, at the clock the
 *    chip holds while doing it, bounds any bf16 kernel on this GPU built on
 *    that instruction.
 *  - HBM streaming: a plain copy (one stream read, one written) and a pass
 *    that reads four streams and writes one (the 4:1 read:write byte mix of
 *    the linear-compression workload), 16-byte accesses, no reuse; and a
 *    read-only pass (the byte mix of a skinny GEMM whose B is streamed once).
 *
 * Conventions: pointers are DEVICE pointers on the current device; the caller
 * owns every buffer; `stream` is a hipStream_t (NULL = the default stream).
 * Calls only enqueue work.  Return value: 0 on success, -1 for an invalid
 * argument (nothing is launched), otherwise the hipError_t of the launch.
 */
#ifndef LLPROBES_H
#define LLPROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* grid workgroups of 4 waves (256 threads), one wave per SIMD; each wave keeps
 * 16 independent 32x32 fp32 accumulators and issues iters x 16 MFMAs of
 * 32x32x16 (32768 flops each): grid * 4 * iters * 16 * 32768 flops per call.
 * operands: NULL (small constant operands, which barely switch the
 * multipliers) or 8 x 256 16-byte fragments of bf16 patterns (32 KiB, 16-byte
 * aligned; fragment f of thread t at (f * 256 + t) * 16 bytes), which every
 * workgroup uses, so that the operands switch as with real data.
 * out: grid * 256 floats (each lane's accumulator sum, so the work is not
 * dead).  grid in [1, 2^20], iters in [0, 2^24]. */
int ll_probe_mfma_only(int grid, int iters, const void* operands, float* out, void* stream);

/* As ll_probe_mfma_only with v_mfma_f32_16x16x32_bf16 (the instruction of
 * the library's 256x256 hand-ordered GEMM kind): each wave keeps 64
 * independent 16x16 accumulators and issues iters x 64 MFMAs of 16384 flops:
 * grid * 4 * iters * 64 * 16384 flops per call (twice ll_probe_mfma_only's
 * at the same iters).  Same arguments, limits and errors. */
int ll_probe_mfma16_only(int grid, int iters, const void* operands, float* out, void* stream);

/* y[i] = x[0][i] ^ x[1][i] ^ ... ^ x[streams-1][i] over n16 16-byte elements
 * per stream: x holds `streams` consecutive arrays of n16 16-byte elements
 * (streams * n16 * 16 bytes read), y holds n16 (n16 * 16 bytes written).
 * streams: 1 (a copy) or 4.  hints: bit 0 non-temporal loads, bit 1
 * non-temporal stores.  x and y 16-byte aligned, not overlapping.
 * grid: workgroups of 256 threads, in [1, 2^20]; n16 >= 0. */
int ll_probe_stream(int streams, int hints, const void* x, void* y, int64_t n16, int grid, void* stream);

/* Read-only streaming: reads x (n16 16-byte elements, n16 * 16 bytes) once;
 * each thread XORs the elements it reads and writes that one 16-byte value
 * to y[thread], so y holds grid * 256 16-byte elements (grid * 4096 bytes
 * written).  hints: 1 non-temporal loads, 0 plain.  x and y 16-byte aligned,
 * not overlapping.  grid in [1, 2^20]; n16 >= 0 (0 still writes y). */
int ll_probe_read(int hints, const void* x, void* y, int64_t n16, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif
