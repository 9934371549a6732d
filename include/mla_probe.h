/*
 * mla_probe.h - measurement probes of the MI355X that the decode's roofline
 * figures are set against: what a plain streaming read and a plain bf16
 * matrix-core loop achieve on the chip, beside the published peaks.  They
 * compute nothing of the attention path.
 *
 * Both launch on `stream` (a hipStream_t; NULL is the null stream) and
 * return without waiting; the caller times them (e.g. with events on the
 * same stream).  Errors: MLA_ERR_NULL for a null required pointer,
 * MLA_ERR_SHAPE for a size out of range, MLA_ERR_HIP when the launch fails.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_probe_stream_read - reads `bytes` bytes of device memory at `src`
 * once, 16 bytes per lane per load with four loads in flight per lane, over
 * 2048 workgroups of 256 lanes.  src: device memory, 16-byte aligned; bytes:
 * a multiple of 16, > 0.  sink: device memory of at least 8192 bytes that
 * the probe may write (its contents carry no meaning; they keep the loads
 * from being removed).  Owns nothing.
 */
mla_status mla_probe_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * mla_probe_mfma_bf16 - `workgroups` workgroups of 4 waves, each wave
 * running `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * accumulations (32 x 32 x 16 bf16 products into float32): 4 * 32768 * iters
 * flops per wave, 16 * 32768 * iters per workgroup.  1 <= iters <= 2^24,
 * 1 <= workgroups <= 2^20.  sink: device memory of at least 4 * workgroups
 * bytes that the probe may write (no meaning; it keeps the products live).
 */
mla_status mla_probe_mfma_bf16(int32_t iters, int32_t workgroups, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
