/*
 * mla_ceilings.h — measured ceilings of the MI355X units the attention
 * kernels of libmla are bound by, for reporting achieved rates as fractions
 * of what the chip delivers beside its published peaks.
 *
 * Each entry point launches one kernel that does only the operation it
 * measures and returns, in *work, the bytes moved or FLOPs issued by that
 * launch; the caller times the launch (events on `stream`) and divides.
 *   - mla_ceiling_hbm_read: a streaming read of `bytes` bytes of `buf`
 *     (16-byte loads, eight in flight per thread, 16 workgroups per compute
 *     unit).  Use a buffer well beyond the 256 MB last-level cache.
 *   - mla_ceiling_mfma_bf16: `iters` rounds of independent bf16 matrix-core
 *     products with fp32 accumulation in every wave, two waves per SIMD;
 *     shape 32x32x16 or 16x16x32 (the two the attention kernels issue).
 *   - mla_ceiling_lds_read: one workgroup per compute unit reading its 128 KB
 *     of LDS back `iters` x 8 times per thread with conflict-free addresses;
 *     kind MLA_CEILING_LDS_B128 (16-byte reads) or MLA_CEILING_LDS_TR_B64
 *     (the transposing 8-byte read of 16-bit elements).
 * Arguments: buf is a device pointer, 16-byte aligned, bytes a positive
 * multiple of 16; sink is a caller-owned device buffer of at least
 * mla_ceiling_sink_floats() floats that receives one value per workgroup
 * (its contents carry no meaning); work may be NULL.  Calls are
 * asynchronous on stream; MLA_ERR_INVALID_ARG for a NULL or misaligned
 * pointer or a bad size, shape or kind; MLA_ERR_HIP for a failed launch.
 */
#ifndef MLA_CEILINGS_H_
#define MLA_CEILINGS_H_

#include <stddef.h>
#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_CEILING_SINK_FLOATS 65536
#define MLA_CEILING_MFMA_32X32X16 0
#define MLA_CEILING_MFMA_16X16X32 1
#define MLA_CEILING_LDS_B128 0
#define MLA_CEILING_LDS_TR_B64 1

int32_t mla_ceiling_sink_floats(void);
mla_status mla_ceiling_hbm_read(const void* buf, size_t bytes, float* sink, double* work, void* stream);
mla_status mla_ceiling_mfma_bf16(int32_t shape, int32_t iters, float* sink, double* work, void* stream);
mla_status mla_ceiling_lds_read(int32_t kind, int32_t iters, float* sink, double* work, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILINGS_H_ */
