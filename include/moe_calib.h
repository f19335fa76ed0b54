/*
 * moe_calib.h -- measurement support exported by the same library as moe.h.
 *
 * Not part of the MoE layer: three kernels whose rates are the on-chip
 * ceilings the layer's kernels are compared with (memory-bound kernels
 * against the copy and streaming-read rates, the grouped GEMM against the
 * MFMA loop), measured on the machine that runs the layer beside the
 * published peaks.  Same conventions as moe.h: device pointers owned by the
 * caller, work enqueued on `stream`, checks before anything is enqueued,
 * MOE_* status codes.
 */
#ifndef MOE_MI355X_CALIB_H
#define MOE_MI355X_CALIB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dst[0 .. bytes) = src[0 .. bytes): 16-byte loads and stores, reads and
 * writes `bytes` each.  src, dst 16-byte aligned device pointers, bytes a
 * multiple of 16; the ranges must not overlap.  bytes = 0 is a no-op.
 */
int moe_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/*
 * Reads src[0 .. bytes) once with 16-byte loads and folds it into one xor,
 * written to *sink (a device word) only if it equals 0x9e3779b9 (pass data
 * that cannot, e.g. zeros).  src 16-byte aligned, bytes a multiple of 16.
 */
int moe_calib_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * `blocks` blocks of four waves; every wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands.  *flops (host)
 * receives the dense bf16 flops enqueued: blocks * 4 * iters * 4 * 32768.
 * sink: one device float, written only on an impossible result.
 */
int moe_calib_mfma(int32_t blocks, int32_t iters, float* sink, double* flops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_CALIB_H */
