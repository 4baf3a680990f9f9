/*
 * lema_measure.h -- measurement and self-check aids exported by liblema.so.
 *
 * These are not part of the optimizer method.  They exist so that the
 * AdamW kernel's bandwidth can be put next to the practical ceiling of the
 * same GPU and so that the arithmetic primitives the kernel is built from
 * can be checked against IEEE results on the host.  Same conventions as
 * lema.h: device pointers, `stream` is a hipStream_t, asynchronous, full
 * validation before any HIP call.
 */
#ifndef LEMA_MEASURE_H
#define LEMA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "lema.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Plain device-to-device copy of `bytes` bytes: one 16-byte vector per lane,
 * one workgroup per 4 KiB, nontemporal loads and stores (the best plain-copy
 * shape measured on MI355X).  Reads `bytes` and writes `bytes`: the
 * read+write bandwidth ceiling, and the known-size reference for HBM byte
 * counters.  src and dst must be 16-byte aligned, bytes a multiple of 16,
 * the ranges disjoint.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP,
 * LEMA_ERR_HIP.
 */
lema_status lema_measure_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Elementwise a/b, sqrt(a) and bf16 nearest-even of a over n elements,
 * compiled exactly as inside the AdamW kernel (same file, same flags).
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_HIP.
 */
lema_status lema_probe_fp32(const float *a, const float *b, float *quot, float *root,
                            uint16_t *bf16, int64_t n, void *stream);

/*
 * r[i] = the reciprocal the int8 kernels take of a row scale s[i] (one Newton
 * step from v_rcp_f32, compiled exactly as in the kernels), for n elements.
 * Their division-free quantization (lema_q8.hip, QuantRow) is exact as long
 * as |r*s - 1| <= 2^-23 for every normal scale, which a test checks over
 * all of them.  Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_ALIGN,
 * LEMA_ERR_HIP.
 */
lema_status lema_probe_q8_reciprocal(const float *s, float *r, int64_t n, void *stream);

/*
 * Counters of the current device's launch-table cache since the library was
 * loaded: out[0] calls that found their table cached, out[1] tables uploaded,
 * out[2] uploads that had to wait for a pending launch, out[3] cached
 * entries.  Launches whose table travels in the kernel arguments (fp32
 * tables of at most 2048 bytes) count in none of them.  Errors:
 * LEMA_ERR_NULL, LEMA_ERR_HIP.
 */
lema_status lema_table_cache_stats(int64_t out[4]);

/* The LDS size per compute unit the current device reports, and the LDS the
 * AdamW step (delta on) reserves per workgroup (the kernel uses none) to cap
 * how many of its workgroups share a CU: 12, or 9 when the step reads
 * `microbatches` >= 4 resident micro-batch gradients (0 = an ordinary step),
 * for launches of 2^18 tiles or more (smaller launches: 16, see
 * lema_step_occupancy kernel 3).  LDS goes to a workgroup in 1280-byte
 * granules on gfx950, so the reservation is a whole number of granules.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE (microbatches < 0), LEMA_ERR_HIP. */
lema_status lema_step_lds_reservation(int32_t microbatches, int32_t *lds_per_cu,
                                      int32_t *reserved_bytes);

/*
 * Residency probe: launches `workgroups` workgroups of `lanes` lanes (a
 * multiple of 64, at most 1024), each with `lds_bytes` of LDS reserved (at
 * most 65536).  The first wavefront of workgroup i stays resident for about
 * `spin_us` microseconds (1 .. 1000) and writes three words to
 * records[3*i .. 3*i+2]: (XCC id << 32) | the HW_ID register (compute unit,
 * shader array and engine bits), then the device wall clock at its start and
 * at its end (hipDeviceAttributeWallClockRate kHz).  The most workgroups
 * that overlapped in time on one compute unit is how many of that size fit
 * there at once.  `records` is device memory of 3 * workgroups words.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_ALIGN, LEMA_ERR_HIP.
 */
lema_status lema_probe_residency(uint64_t *records, int32_t workgroups, int32_t lanes,
                                 int32_t lds_bytes, int32_t spin_us, void *stream);

/*
 * The occupancy plan of a step kernel on the current device, for checking
 * with lema_probe_residency.  `kernel`:
 *   0  the fp32 AdamW step (bf16 gradient, delta on), launches of 2^18
 *      tiles or more
 *   1  the fp32 step on 8 resident bf16 micro-batches (delta on)
 *   2  the int8-moment step, 256-lane wave-row workgroups (bf16 gradient,
 *      delta on)
 *   3  the fp32 AdamW step in launches of fewer than 2^18 tiles
 * out[0] lanes per workgroup, out[1] the kernel's static LDS bytes, out[2]
 * the dynamic LDS bytes a launch reserves, out[3] the workgroups per CU the
 * reservation is meant to allow, out[4] the workgroups per CU its registers
 * and static LDS alone allow (hipOccupancyMaxActiveBlocksPerMultiprocessor),
 * out[5] the LDS allocation granule the reservation assumes.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE (unknown kernel), LEMA_ERR_HIP.
 */
lema_status lema_step_occupancy(int32_t kernel, int32_t out[6]);

/* Compute units of the current device and the elements one workgroup takes
 * per tile in the AdamW and accumulation kernels. */
lema_status lema_device_info(int32_t *compute_units, int32_t *tile_elements);

#ifdef __cplusplus
}
#endif

#endif /* LEMA_MEASURE_H */
