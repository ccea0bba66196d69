/*
 * pa_measure.h -- measurement aid shipped with the paged decode-attention
 * library (AMD MI355X, gfx950).  Not part of the attention method: it gives
 * the bandwidth a plain streaming read attains on the device the decode runs
 * on, so that the decode's achieved HBM bandwidth can be reported against
 * both the published peak and what a read with nothing else to do reaches,
 * measured in the same process.
 *
 * Same conventions as pagedattn.h: device pointers owned by the caller,
 * asynchronous on `stream`, arguments checked on the host, status codes,
 * no allocation and no state between calls.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_stream_read -- read `bytes` bytes of device memory at `src` exactly
 * once, with 16-byte non-temporal loads (the decode's tile loads), every
 * workgroup streaming one contiguous share of the buffer, eight loads in
 * flight per lane, over a grid of 8 workgroups of 256 threads per compute
 * unit of the current device.  Nothing is written except, in the
 * vanishingly rare case that the XOR of a workgroup's data equals a fixed
 * constant, that value to *sink -- the condition keeps the loads from being
 * optimised away; the value means nothing.
 *
 *   src    device pointer, 16-byte aligned
 *   bytes  a multiple of 16; 0 does nothing
 *   sink   device pointer to one uint32_t
 *
 * Errors: PA_ERR_INVALID_ARG for a null or misaligned pointer or a size
 * that is not a multiple of 16; PA_ERR_HIP when the device cannot be
 * queried or the launch fails.
 */
pa_status pa_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H */
