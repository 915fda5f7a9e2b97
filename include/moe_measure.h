/*
 * moe_measure.h -- measurement helpers, libmoe_measure.so.
 *
 * Not part of the MoE layer and not linked into libmoe.so: two kernels that
 * measure what one MI355X delivers beside its published peaks (HBM read
 * bandwidth, dense bf16 matrix-core throughput), so that a layer's roofline
 * fraction can be read against the spec sheet and against the measured
 * ceiling.  Same conventions as moe.h: device pointers, `stream` a
 * hipStream_t passed as void* (NULL = null stream), asynchronous, int status
 * with a caller-provided message buffer (truncated to err_len, NUL-terminated;
 * nothing is enqueued on error).
 */
#ifndef MOE_MEASURE_H
#define MOE_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_MEASURE_OK = 0,
    MOE_MEASURE_EINVAL = -1,   /* bad size, NULL or misaligned pointer */
    MOE_MEASURE_EHIP = -3      /* HIP launch error */
};

/* The matrix-core ceiling.  Each CU runs eight waves of iters x 8 independent
 * bf16 MFMAs (32x32x16, fp32 accumulate) with no memory traffic; one float per
 * wave is written to sink (device, 16-byte aligned, at least 32 bytes per CU:
 * sink_bytes is checked).  clock (device, 2 x uint64, 8-byte aligned, or NULL)
 * receives block 0's shader-clock cycles and 100 MHz ticks over the loop
 * (their ratio is the shader clock).  *flops (host, or NULL) receives the
 * launch's floating-point operation count; the caller times the launch.
 * MOE_MEASURE_EINVAL for iters outside [1, 2^24], a NULL or misaligned sink, a
 * short sink or a misaligned clock. */
int moe_mfma_ceiling(int32_t iters, float *sink, size_t sink_bytes, uint64_t *clock,
                     int64_t *flops, void *stream, char *err, size_t err_len);

/* The HBM read ceiling: reads `bytes` of device memory at buf once with plain
 * streaming 16-byte loads (one 256-thread block per CU, each wave on
 * contiguous 8 KB runs) and XORs every 32-bit word into *sink (device,
 * 4-byte aligned, caller-initialised).  bytes a multiple of 16, buf 16-byte
 * aligned (may be NULL when bytes is 0).  MOE_MEASURE_EINVAL otherwise. */
int moe_read_ceiling(const void *buf, size_t bytes, uint32_t *sink, void *stream, char *err,
                     size_t err_len);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MEASURE_H */
