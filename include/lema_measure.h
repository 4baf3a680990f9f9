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
 * entries.  Errors: LEMA_ERR_NULL, LEMA_ERR_HIP.
 */
lema_status lema_table_cache_stats(int64_t out[4]);

/* The LDS size per compute unit the current device reports, and the LDS the
 * AdamW step reserves per workgroup (the kernel uses none) to cap how many of
 * its workgroups share a CU: about 13, or 10 when the step reads
 * `microbatches` >= 4 resident micro-batch gradients (0 = an ordinary step).
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE (microbatches < 0), LEMA_ERR_HIP. */
lema_status lema_step_lds_reservation(int32_t microbatches, int32_t *lds_per_cu,
                                      int32_t *reserved_bytes);

/* Compute units of the current device and the elements one workgroup takes
 * per tile in the AdamW and accumulation kernels. */
lema_status lema_device_info(int32_t *compute_units, int32_t *tile_elements);

#ifdef __cplusplus
}
#endif

#endif /* LEMA_MEASURE_H */
