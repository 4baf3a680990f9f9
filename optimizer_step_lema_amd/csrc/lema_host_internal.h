// lema_host_internal.h -- host helpers shared by the C ABI translation units.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <functional>
#include <vector>

#include "lema.h"
#include "lema_internal.h"

namespace lema {

// Tile counts of one call stay below this, so that 32-bit tile indices plus
// a launch's grid never wrap.
constexpr uint64_t kMaxTiles = (uint64_t(1) << 32) - (uint64_t(1) << 20);

// Address range [lo, hi) of one array in one call; `written` if the call
// stores into it.
struct Span {
    uintptr_t lo, hi;
    bool written;
};

// Records hipError_t `e` as this thread's last HIP error; returns LEMA_ERR_HIP.
lema_status hip_failed(hipError_t e);

// Hyperparameters and gradient dtype (LEMA_GRAD_Q8 only where allowed).
lema_status check_hparams(const lema_adamw_args *a, bool allow_q8_grad = false);
AdamwConsts derive_consts(const lema_adamw_args *a);

// Spans kept in storage the caller provides, for a call that allocates
// nothing: a span beyond `cap` sets `overflow` instead of being stored.
struct FixedSpans {
    Span *data;
    size_t cap;
    size_t n = 0;
    bool overflow = false;
    void push_back(const Span &s) {
        if (n < cap)
            data[n++] = s;
        else
            overflow = true;
    }
};

// Validates segment descriptors (sizes, pairing, required pointers,
// element alignment) and appends their spans when `spans` is non-null.
lema_status validate_adamw_segs(const lema_adamw_seg *segs, int32_t nseg, int32_t grad_dtype,
                                bool delta_allowed, std::vector<Span> *spans);
lema_status validate_adamw_segs(const lema_adamw_seg *segs, int32_t nseg, int32_t grad_dtype,
                                bool delta_allowed, FixedSpans *spans);
// True if two spans intersect and at least one of them is written (sorts
// the spans in place; allocates nothing).
bool any_conflict(Span *begin, Span *end);
bool any_conflict(std::vector<Span> &spans);
void add_span(std::vector<Span> &spans, const void *p, int64_t numel, size_t elem, bool written);

// Validates int8-path segment descriptors for a gradient dtype and moment
// dtype: sizes, row lengths (when an array is int8), required pointers,
// element alignment, and delta only where allowed.  Appends the arrays'
// spans when `spans` is non-null and the launch records of the non-empty
// segments when `recs` is non-null; sets *with_delta when a segment writes a
// delta.
lema_status validate_q8_segs(const lema_adamw_q8_seg *segs, int32_t nseg, int32_t grad_dtype,
                             int32_t moment_dtype, bool delta_allowed, std::vector<Span> *spans,
                             std::vector<Q8Rec> *recs, bool *with_delta);
// Rows of a tensor of numel elements cut into rows of row_len.
int64_t q8_rows(int64_t numel, int64_t row_len);

// Launch records of the non-empty segments; last_bf16 (may be NULL) gives
// each segment's last micro-batch for the fused accumulate-and-step mode.
void adamw_records(const lema_adamw_seg *segs, int32_t nseg, std::vector<SegRec> *out,
                   const uint16_t *const *last_bf16);

// Run launch(device copy of `bytes`) on the per-device table cache: the
// table is uploaded unless a byte-identical one is cached, and stays
// reserved until the launched work on `stream` has finished.  `launch` runs
// with the device's cache locked: it must not call anything that takes that
// lock again (device state, occupancy_lds_bytes, another launch_on_table).
lema_status launch_on_table(const std::vector<unsigned char> &bytes, hipStream_t stream,
                            const std::function<hipError_t(const void *)> &launch);

// Launch through the per-device table cache on `stream`.
lema_status launch_adamw_recs(const std::vector<SegRec> &recs, const AdamwConsts &c,
                              GradMode grad_mode, hipStream_t stream);
lema_status launch_accum_recs(const std::vector<SegRec> &recs, bool overwrite,
                              hipStream_t stream);
// kGradBf16Sum: `lists` holds each record's `nmb` micro-batch pointers in
// record order; they are appended to the table and the records point there.
lema_status launch_adamw_sum_recs(std::vector<SegRec> recs, const std::vector<uint64_t> &lists,
                                  int nmb, const AdamwConsts &c, hipStream_t stream);
lema_status launch_merge_recs(const std::vector<SegRec> &recs, hipStream_t stream);

// Dynamic LDS to reserve per workgroup of kernel `fn` so that at most
// `workgroups_per_cu` of them share a CU of the current device: the
// kernel's static LDS is subtracted and the total kept to whole allocation
// granules (0 if the device or the kernel cannot be queried).
uint32_t occupancy_lds_bytes(const void *fn, int workgroups_per_cu);
// Workgroups of `lanes` lanes of kernel `fn` that its registers and static
// LDS alone let share a CU (0 if the runtime cannot tell); cached per kernel.
int register_occupancy(const void *fn, int lanes);
// Compute units of the current device (0 if it cannot be queried).
int compute_units();
// Workgroups of the fp32 AdamW step allowed per CU when it reads `nmb`
// resident micro-batches (0 for the other gradient modes) in a launch of
// `tiles` tiles, and the dynamic LDS its kernel reserves for that.
int step_workgroups_per_cu(int nmb, uint64_t tiles);
uint32_t step_lds_bytes_for(GradMode grad_mode, bool with_delta, int nmb, uint64_t tiles);

}  // namespace lema
