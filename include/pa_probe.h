/*
 * pa_probe.h - measurement aid of libpagedattn: a plain streaming read of
 * device memory, the achievable read bandwidth that the decode kernels'
 * HBM figures are compared with.  Not part of the attention path.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_probe_stream_read - read `bytes` of device memory once.
 *
 * Each of `workgroups` workgroups of 512 lanes reads 64 KiB slices of `src`
 * (16-byte non-temporal loads, eight per lane in flight) in a grid-stride
 * loop and writes the XOR of everything it read, 16 bytes, to sink[its
 * index].  Only workgroups dealt to the XCDs whose bits are set in
 * `xcd_mask` (bit x: XCD x = workgroup index mod 8) read; the others write
 * zeros, so a mask of a few XCDs shows what they pull on their own.
 *
 *   src         DEVICE, 16-byte aligned, `bytes` readable
 *   bytes       a multiple of 65536 (0 enqueues nothing)
 *   workgroups  8 .. 2^20; the workgroups past the last multiple of 8 read
 *               nothing, so every XCD has the same count
 *   xcd_mask    bits 0..7, at least one set
 *   sink        DEVICE, 16-byte aligned, 16 * workgroups bytes, written
 *   stream      hipStream_t (NULL = null stream)
 * Returns PA_ERR_NULL, PA_ERR_SHAPE (misaligned, bad sizes, host memory) or
 * PA_ERR_LAUNCH; PA_OK when enqueued.
 */
int pa_probe_stream_read(const void *src, size_t bytes, int32_t workgroups, int32_t xcd_mask,
                         void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
