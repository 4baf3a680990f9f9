// lema_internal.h -- interface between the host layer and the gfx950 kernels.
// Not installed; the public ABI is include/lema.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lema {

// Work decomposition.  A tile is the unit one workgroup processes: kBlock
// lanes x kVec contiguous elements x kUnroll accesses per lane.  Each access
// moves 16 bytes of every fp32 array and 8 bytes of every bf16 array per
// lane, contiguous across the wavefront.  One wavefront per workgroup and one
// access per lane measured fastest on MI355X for this 9-11-stream pattern
// (5.95 TB/s against 5.71 for 256 lanes x 2 and 5.40 for 512 lanes x 1).
constexpr int kBlock = 64;
constexpr int kVec = 4;
constexpr int kUnroll = 1;
constexpr int64_t kTile = int64_t(kBlock) * kVec * kUnroll;   // 256 elements
// A launch's grid holds at most 2^31 work-items (the dispatch packet counts
// work-items in 32 bits); larger grids are split into consecutive launches.
// For the 64-lane tile kernels that is 2^25 tiles (8.6 G elements), so a
// step over a whole 7B-parameter model is one launch.
constexpr uint32_t kMaxWorkItemsPerLaunch = 1u << 31;
constexpr uint32_t max_blocks_per_launch(int lanes) {
    return kMaxWorkItemsPerLaunch / uint32_t(lanes);
}

// One segment of the launch table: up to eight array pointers and the length.
//   AdamW : p = {master, m, v, grad, weight_bf16, orig_bf16, delta, last_bf16}
//   accum : p = {acc, grad_bf16, 0, 0, 0, 0, 0, 0}
//   merge : p = {base_bf16, delta, merged_bf16, 0, 0, 0, 0, 0}
struct SegRec {
    uint64_t p[8];
    int64_t numel;
    int64_t reserved;
};
static_assert(sizeof(SegRec) == 80, "segment record is 80 bytes");

// How the AdamW kernel reads the gradient.
enum GradMode : int {
    kGradBf16 = 0,         // grad: bf16 bits of one micro-batch
    kGradF32 = 1,          // grad: the fp32 accumulator
    kGradF32PlusBf16 = 2,  // grad: fp32 accumulator + f32(last bf16 micro-batch)
    kGradBf16Sum = 3,      // grad: fp32 sum, in order, of K bf16 micro-batches
};

// kGradBf16Sum records: p[3] is the byte offset, from the start of the launch
// table, of the segment's K micro-batch pointers (uint64 each, appended after
// the records); p[7] is the OR of those pointers (for the alignment test);
// `reserved` is K.
constexpr int kMaxMicrobatches = 16;

// The launch table in device memory is
//   uint32_t tile_begin[nseg + 1]   (prefix sum of tiles per segment)
//   padding to a multiple of 64 bytes
//   SegRec   rec[nseg]
constexpr size_t table_tiles_bytes(int nseg) {
    return (sizeof(uint32_t) * (size_t(nseg) + 1) + 63) & ~size_t(63);
}
constexpr size_t table_bytes(int nseg) {
    return table_tiles_bytes(nseg) + sizeof(SegRec) * size_t(nseg);
}

// A launch table of at most kInlineTableBytes can travel by value in the
// kernel arguments of the fp32 tile kernels (adamw, accum, merge) instead of
// through a device copy: up to 24 segments, or a one-layer kGradBf16Sum
// table with its micro-batch lists.  Such a launch needs no table upload,
// no cache entry and no event recording when the cache may reuse the copy;
// on MI355X that event alone cost about 3 us of GPU time per launch of
// back-to-back steps.
constexpr size_t kInlineTableBytes = 2048;
struct InlineTable {
    uint64_t w[kInlineTableBytes / 8];
};

// ------------------------------------------------ int8 rows with scales
//
// The int8 kernels give each row to a team of 2^team_log2 lanes of one
// workgroup; every lane holds up to `chunks` chunks of 4 consecutive row
// elements in registers.  Workgroups have kQBlock lanes and hold up to
// kQStepChunks (AdamW) or kQCodeChunks (accumulation, conversions) chunks per
// lane; rows too long for that go to kQBlockWide-lane workgroups with
// kQWideChunks per lane.  The launch table has the layout above with Q8Rec
// records, and its prefix sums count workgroups.
constexpr int kQBlock = 256;
constexpr int kQBlockWide = 1024;
// Four chunks (16 elements) per lane measured fastest for both families on
// MI355X: 8 or 16 per lane cut occupancy more than they add loads in flight
// (int8 step 5.50 TB/s at 4, 4.97 at 8, 2.47 at 16 with 256 VGPRs;
// accumulation 4.0 TB/s at 4, 1.7 at 8, 2.5 at 16).
constexpr int kQStepChunks = 4;
constexpr int kQ8StepWorkgroupsPerCu = 3;     // occupancy cap of the 256-lane step
constexpr int kQCodeChunks = 4;
constexpr int kQWideChunks = 4;
// Wave-row accumulation and conversions hold up to 16 chunks per lane in
// kQBlock-lane workgroups, which covers every row up to kQMaxRow there: on
// MI355X rows of 11,008 ran 26% faster as 256-lane teams with 11 chunks than
// as 1024-lane teams with 3 (four or five rows per CU instead of two), and
// rows of 4096 as well as one wavefront with 16 chunks as four with 4.  The
// step keeps 4 (its lanes hold more state per chunk).
constexpr int kQWaveCodeChunks = 16;
constexpr int64_t kQMaxRow = int64_t(kQBlockWide) * kQWideChunks * 4;   // 16384 elements

struct Q8Rec {
    // step        : {master, m, m_scale, v, v_scale, grad, grad_scale, weight, orig, delta}
    // accumulation: {acc_codes, acc_scale, grad_bf16}
    // quantize    : {x, codes, scale}
    uint64_t p[10];
    int64_t numel;
    int64_t row_len;
    int64_t rows;
    int32_t team_log2;    // lanes per row = 1 << team_log2, at most the workgroup
    int32_t chunks;       // 4-element chunks per lane
    int32_t flags;        // kQVector: full chunks take 16/8/4-byte vector accesses;
                          // kQPacked: packed rows; kQWave: wave rows
    int32_t block;        // lanes of the workgroups the record is sized for
};
static_assert(sizeof(Q8Rec) == 120, "int8 segment record is 120 bytes");
constexpr int32_t kQVector = 1;
// Rows of 4*2^team_log2 elements (4 .. 256) on vector-aligned arrays: every
// chunk of a lane belongs to its own row, `chunks` rows per lane, so that a
// wavefront's chunk steps stay contiguous (lema_q8.hip, packed rows).
constexpr int32_t kQPacked = 2;
// Rows whose team spans whole wavefronts (team_log2 >= 6) on vector-aligned
// arrays with a multiple-of-4 element count: every wavefront works on one
// row, reached through row-sized buffer resources (lema_q8.hip, wave rows).
constexpr int32_t kQWave = 4;

// Kernel family of a launch group: row teams, packed rows or wave rows; or,
// for the step, mixed: packed-row and wave-row records in one launch of
// kQBlock-lane workgroups, each workgroup taking its record's path, with
// wave rows of up to kQMixedWaveChunks chunks per lane (rows of up to
// 11,264 elements, which other launches put in kQBlockWide-lane
// workgroups).  11 chunks keep the mixed kernel at 167 VGPRs or fewer for
// the common gradient kinds, within the 3 workgroups per CU of the step's
// occupancy cap; 12 took it to 178.  One launch lets the families' workgroups fill each other's
// tails instead of running one group after another.
enum QRows : int { kQRowsTeam = 0, kQRowsPacked = 1, kQRowsWave = 2, kQRowsMixed = 3 };
constexpr int kQMixedWaveChunks = 11;
// Records of a mixed launch carry this flag (with kQPacked or kQWave).
constexpr int32_t kQMixed = 8;

// How the int8 step reads the moments and the gradient.
enum QGrad : int { kQGradBf16 = 0, kQGradF32 = 1, kQGradQ8 = 2 };

constexpr size_t q8_table_bytes(int nseg) {
    return table_tiles_bytes(nseg) + sizeof(Q8Rec) * size_t(nseg);
}

struct AdamwConsts {
    float b1, omb1, b2, omb2, eps, decay, step_size, inv_bc2_root;
};

// Kernel launches (asynchronous on `stream`).  The launch table is `table`,
// a device copy, when that is not null, else `*inl`, copied into the kernel
// arguments; one workgroup runs per tile 0 .. total_tiles-1.
// `nmb` is the micro-batch count of kGradBf16Sum (ignored otherwise).
// `lds_bytes` of LDS are reserved per workgroup of the AdamW kernel, which
// itself uses none: the reservation caps how many of its workgroups share a
// CU.
hipError_t launch_adamw(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, GradMode grad_mode, bool with_delta,
                        const AdamwConsts &c, hipStream_t stream, int nmb, uint32_t lds_bytes);
hipError_t launch_accum(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, bool overwrite, hipStream_t stream);
hipError_t launch_merge(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, hipStream_t stream);

// int8 kernels; `block` (kQBlock or kQBlockWide) is the workgroup size the
// table's records were sized for, `rows` the kernel family of all its records
// (packed rows: kQBlock only).  The step reserves `lds_bytes` of unused LDS
// per workgroup, a cap on its workgroups per CU.
hipError_t launch_adamw_q8(const void *table, int nseg, uint32_t total_blocks, bool moments_q8,
                           QGrad grad, bool with_delta, int block, QRows rows,
                           const AdamwConsts &c, hipStream_t stream, uint32_t lds_bytes);
hipError_t launch_accum_q8(const void *table, int nseg, uint32_t total_blocks, bool overwrite,
                           int block, QRows rows, hipStream_t stream);
hipError_t launch_quantize_q8(const void *table, int nseg, uint32_t total_blocks, bool dequantize,
                              int block, QRows rows, hipStream_t stream);

// The kernel functions launch_adamw and launch_adamw_q8 run for these
// arguments (nullptr where they would refuse them): occupancy planning
// queries their static LDS and registers.
const void *adamw_kernel_fn(GradMode grad_mode, bool with_delta, int nmb);
const void *adamw_q8_kernel_fn(bool moments_q8, QGrad grad, bool with_delta, int block,
                               QRows rows);

// Measurement aids (include/lema_measure.h).
hipError_t launch_residency_probe(uint64_t *rec, int workgroups, int lanes, uint32_t lds_bytes,
                                  uint64_t ticks, hipStream_t stream);
hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);
hipError_t launch_fp32_probe(const float *a, const float *b, float *quot,
                             float *root, uint16_t *bf16, int64_t n,
                             hipStream_t stream);
hipError_t launch_q8_recip_probe(const float *s, float *r, int64_t n, hipStream_t stream);

}  // namespace lema
