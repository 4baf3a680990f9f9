// lema_kernels.hip -- gfx950 kernels of the mixed-precision AdamW path.
//
// adamw_tile_kernel : one AdamW step over a list of segments (LEMA README,
//   "Quick Start": torch.optim.AdamW; "Selective Full Fine-Tuning": per-layer
//   AdamW over fp32 master, m and v, fp32 delta for checkpoints; LLMScale
//   fine-tuning VRAM page: bf16 weight and gradient next to fp32 states).
// accum_tile_kernel : fp32 accumulation of a bf16 micro-batch gradient
//   (README, "Selective Full Fine-Tuning": fp32 gradient accumulation).
// merge_tile_kernel : servable bf16 weight from base + saved fp32 delta
//   (README, "Selective Full Fine-Tuning": merge_delta).
//
// Both are elementwise and bound by HBM bandwidth, so there is no MFMA and
// no LDS tiling of data: each lane streams 4 contiguous elements per access
// (16-byte fp32 / 8-byte bf16 vector loads and stores, contiguous across the
// wavefront).  The accesses go through per-tile buffer resources with the
// nontemporal hint, since no byte is touched twice (lema_device.h).
//
// One workgroup per tile, not a persistent grid: on gfx9 the vector-memory
// counter also counts stores, so a persistent loop would wait for a tile's
// stores before its next loads could be waited on; short-lived workgroups
// leave their stores in flight and a fresh workgroup takes the CU slot.  The
// tiles of all segments are numbered consecutively; a workgroup finds its
// segment by a binary search over the tile prefix sums of the launch table
// (wave-uniform, so it runs on scalar loads that hit the scalar cache) and
// reads the segment's record with one scalar load.
//
// Arithmetic: binary32 only, no contraction into FMA (this file is built with
// -ffp-contract=off and every arithmetic function also carries the pragma),
// correctly rounded sqrt and division (the compiler's IEEE expansions),
// subnormals kept, bf16 output rounded to nearest even by gfx950's
// v_cvt_pk_bf16_f32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>

#include "lema_device.h"
#include "lema_internal.h"

namespace lema {
namespace {

using namespace dev;

// ------------------------------------------------------------- AdamW

// kNmb: the number of micro-batches of kGradBf16Sum (a compile-time count,
// so that all their loads issue back to back); 0 for the other modes.
template <GradMode kMode, bool kDelta, int kNmb>
struct AdamwTile {
    AdamwConsts c;
    ktable_t table;      // the launch table (micro-batch pointer lists live there)

    __device__ __forceinline__ void operator()(const SegRec &r, uint32_t local_tile) const {
        const uint64_t master = r.p[0], m = r.p[1], v = r.p[2], grad = r.p[3];
        const uint64_t weight = r.p[4], orig = r.p[5], delta = r.p[6], last = r.p[7];
        const int64_t numel = r.numel;
        const int64_t base = int64_t(local_tile) * kTile;

        constexpr bool kGradIsF32 = kMode == kGradF32 || kMode == kGradF32PlusBf16;
        const bool has_delta = kDelta && delta != 0;
        const uint64_t fp32_bits = master | m | v | (kGradIsF32 ? grad : 0) | (has_delta ? delta : 0);
        const uint64_t bf16_bits = (kMode == kGradBf16 ? grad : 0) | weight | (has_delta ? orig : 0) |
                                   (kMode == kGradF32PlusBf16 || kMode == kGradBf16Sum ? last : 0);
        const bool vector_ok = base + kTile <= numel && (fp32_bits & 15) == 0 && (bf16_bits & 7) == 0;

        if (vector_ok) {
            if (has_delta)
                vector_tile<true>(master, m, v, grad, last, weight, orig, delta, base);
            else
                vector_tile<false>(master, m, v, grad, last, weight, orig, delta, base);
        } else {
            element_tile(master, m, v, grad, last, weight, has_delta ? orig : 0,
                         has_delta ? delta : 0, base, numel);
        }
    }

    // The K micro-batch pointers of a kGradBf16Sum segment.
    __device__ __forceinline__ const LEMA_CONST uint64_t *microbatches(uint64_t list_offset) const {
        return (const LEMA_CONST uint64_t *)(table + list_offset);
    }

    // The gradient of this lane's 4 elements of the tile whose first vector
    // index is q0.
    __device__ __forceinline__ f32x4 load_grad4(uint64_t grad, uint64_t last, int64_t q0,
                                                int lane) const {
#pragma clang fp contract(off)
        if constexpr (kMode == kGradBf16) {
            const u32x2 gb = tile_ld<u32x2>(tile_rsrc<u32x2>(grad, q0, kBlock), lane);
            return f32x4{bf16_lo(gb.x), bf16_hi(gb.x), bf16_lo(gb.y), bf16_hi(gb.y)};
        } else if constexpr (kMode == kGradF32) {
            return tile_ld<f32x4>(tile_rsrc<f32x4>(grad, q0, kBlock), lane);
        } else if constexpr (kMode == kGradBf16Sum) {
            // every micro-batch's loads first, then the fp32 sum in micro-batch
            // order, the first one widened exactly (lema_grad_accum's overwrite)
            const LEMA_CONST uint64_t *mb = microbatches(grad);
            u32x2 gb[kNmb];
#pragma unroll
            for (int k = 0; k < kNmb; ++k) gb[k] = tile_ld<u32x2>(tile_rsrc<u32x2>(mb[k], q0, kBlock), lane);
            f32x4 acc = {bf16_lo(gb[0].x), bf16_hi(gb[0].x), bf16_lo(gb[0].y), bf16_hi(gb[0].y)};
#pragma unroll
            for (int k = 1; k < kNmb; ++k) {
                acc = f32x4{accum_elem(acc.x, bf16_lo(gb[k].x), false),
                            accum_elem(acc.y, bf16_hi(gb[k].x), false),
                            accum_elem(acc.z, bf16_lo(gb[k].y), false),
                            accum_elem(acc.w, bf16_hi(gb[k].y), false)};
            }
            return acc;
        } else {
            // the last micro-batch's fp32 addition, as lema_grad_accum does it
            const f32x4 acc = tile_ld<f32x4>(tile_rsrc<f32x4>(grad, q0, kBlock), lane);
            const u32x2 lb = tile_ld<u32x2>(tile_rsrc<u32x2>(last, q0, kBlock), lane);
            return f32x4{accum_elem(acc.x, bf16_lo(lb.x), false), accum_elem(acc.y, bf16_hi(lb.x), false),
                         accum_elem(acc.z, bf16_lo(lb.y), false), accum_elem(acc.w, bf16_hi(lb.y), false)};
        }
    }

    template <bool kHasDelta>
    __device__ __forceinline__ void vector_tile(uint64_t master, uint64_t m, uint64_t v,
                                                uint64_t grad, uint64_t last, uint64_t weight,
                                                uint64_t orig, uint64_t delta, int64_t base) const {
        f32x4 w4[kUnroll], m4[kUnroll], v4[kUnroll], g4[kUnroll];
        u32x2 o2[kUnroll];
        const int lane = int(threadIdx.x);

        // all loads of the tile first, so each lane has them in flight together
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;   // first vector of the access
            w4[u] = tile_ld<f32x4>(tile_rsrc<f32x4>(master, q0, kBlock), lane);
            m4[u] = tile_ld<f32x4>(tile_rsrc<f32x4>(m, q0, kBlock), lane);
            v4[u] = tile_ld<f32x4>(tile_rsrc<f32x4>(v, q0, kBlock), lane);
            g4[u] = load_grad4(grad, last, q0, lane);
            if constexpr (kHasDelta) o2[u] = tile_ld<u32x2>(tile_rsrc<u32x2>(orig, q0, kBlock), lane);
        }

#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;
            f32x4 w = w4[u], mm = m4[u], vv = v4[u];
            const f32x4 g = g4[u];
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                float wk = w[k], mk = mm[k], vk = vv[k];
                adamw_elem(wk, mk, vk, g[k], c);
                w[k] = wk;
                mm[k] = mk;
                vv[k] = vk;
            }
            tile_st<f32x4>(tile_rsrc<f32x4>(master, q0, kBlock), lane, w);
            tile_st<f32x4>(tile_rsrc<f32x4>(m, q0, kBlock), lane, mm);
            tile_st<f32x4>(tile_rsrc<f32x4>(v, q0, kBlock), lane, vv);
            tile_st<u32x2>(tile_rsrc<u32x2>(weight, q0, kBlock), lane,
                           u32x2{to_bf16_pair(w.x, w.y), to_bf16_pair(w.z, w.w)});
            if constexpr (kHasDelta) {
#pragma clang fp contract(off)
                const u32x2 o = o2[u];
                const f32x4 d = {w.x - bf16_lo(o.x), w.y - bf16_hi(o.x),
                                 w.z - bf16_lo(o.y), w.w - bf16_hi(o.y)};
                tile_st<f32x4>(tile_rsrc<f32x4>(delta, q0, kBlock), lane, d);
            }
        }
    }

    // Partial tiles and segments whose arrays are not vector-aligned: one
    // element at a time, same lane-to-element map as the vector path.
    __device__ __forceinline__ void element_tile(uint64_t master, uint64_t m, uint64_t v,
                                                 uint64_t grad, uint64_t last, uint64_t weight,
                                                 uint64_t orig, uint64_t delta, int64_t base,
                                                 int64_t numel) const {
#pragma clang fp contract(off)
        const int64_t lane = int64_t(threadIdx.x) * kVec;
        for (int u = 0; u < kUnroll; ++u) {
            for (int k = 0; k < kVec; ++k) {
                const int64_t e = base + u * (kBlock * kVec) + lane + k;
                if (e >= numel) continue;
                float g;
                if constexpr (kMode == kGradBf16)
                    g = bf16_one(as_global<gu16>(grad)[e]);
                else if constexpr (kMode == kGradF32)
                    g = as_global<gfloat>(grad)[e];
                else if constexpr (kMode == kGradBf16Sum) {
                    const LEMA_CONST uint64_t *mb = microbatches(grad);
                    g = bf16_one(as_global<gu16>(mb[0])[e]);
                    for (int j = 1; j < kNmb; ++j)
                        g = accum_elem(g, bf16_one(as_global<gu16>(mb[j])[e]), false);
                } else
                    g = accum_elem(as_global<gfloat>(grad)[e], bf16_one(as_global<gu16>(last)[e]), false);
                float w = as_global<gfloat>(master)[e];
                float mm = as_global<gfloat>(m)[e];
                float vv = as_global<gfloat>(v)[e];
                adamw_elem(w, mm, vv, g, c);
                as_global<gfloat>(master)[e] = w;
                as_global<gfloat>(m)[e] = mm;
                as_global<gfloat>(v)[e] = vv;
                as_global<gu16>(weight)[e] = to_bf16_one(w);
                if (delta != 0) as_global<gfloat>(delta)[e] = w - bf16_one(as_global<gu16>(orig)[e]);
            }
        }
    }
};

template <GradMode kMode, bool kDelta, int kNmb = 0>
__global__ __launch_bounds__(kBlock) void adamw_tile_kernel(const void *table, int nseg,
                                                            uint32_t tile0, AdamwConsts c,
                                                            InlineTable inl) {
    const ktable_t t = launch_table(table, inl);
    block_of_table<SegRec>(t, nseg, tile0, AdamwTile<kMode, kDelta, kNmb>{c, t});
}

template <int kNmb>
const void *sum_kernel(bool with_delta) {
    return with_delta ? reinterpret_cast<const void *>(&adamw_tile_kernel<kGradBf16Sum, true, kNmb>)
                      : reinterpret_cast<const void *>(&adamw_tile_kernel<kGradBf16Sum, false, kNmb>);
}

// The kGradBf16Sum kernel for nmb micro-batches (1 .. kMaxMicrobatches).
template <std::size_t... I>
const void *pick_sum_kernel(int nmb, bool with_delta, std::index_sequence<I...>) {
    const void *fns[] = {sum_kernel<int(I) + 1>(with_delta)...};
    return fns[nmb - 1];
}

// ------------------------------------------------------ accumulation

template <bool kOverwrite>
struct AccumTile {
    __device__ __forceinline__ void operator()(const SegRec &r, uint32_t local_tile) const {
        const uint64_t acc = r.p[0], g = r.p[1];
        const int64_t numel = r.numel;
        const int64_t base = int64_t(local_tile) * kTile;
        const int64_t lane = int64_t(threadIdx.x) * kVec;
        const bool vector_ok = base + kTile <= numel && (acc & 15) == 0 && (g & 7) == 0;

        if (vector_ok) {
            f32x4 a4[kUnroll];
            u32x2 g2[kUnroll];
            const int vl = int(threadIdx.x);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;
                if constexpr (!kOverwrite) a4[u] = tile_ld<f32x4>(tile_rsrc<f32x4>(acc, q0, kBlock), vl);
                g2[u] = tile_ld<u32x2>(tile_rsrc<u32x2>(g, q0, kBlock), vl);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;
                const f32x4 gf = {bf16_lo(g2[u].x), bf16_hi(g2[u].x), bf16_lo(g2[u].y),
                                  bf16_hi(g2[u].y)};
                f32x4 out;
                if constexpr (kOverwrite) {
                    out = gf;
                } else {
#pragma unroll
                    for (int k = 0; k < kVec; ++k) out[k] = accum_elem(a4[u][k], gf[k], false);
                }
                tile_st<f32x4>(tile_rsrc<f32x4>(acc, q0, kBlock), vl, out);
            }
        } else {
            for (int u = 0; u < kUnroll; ++u) {
                for (int k = 0; k < kVec; ++k) {
                    const int64_t e = base + u * (kBlock * kVec) + lane + k;
                    if (e >= numel) continue;
                    const float ge = bf16_one(as_global<gu16>(g)[e]);
                    as_global<gfloat>(acc)[e] =
                        kOverwrite ? ge : accum_elem(as_global<gfloat>(acc)[e], ge, false);
                }
            }
        }
    }
};

template <bool kOverwrite>
__global__ __launch_bounds__(kBlock) void accum_tile_kernel(const void *table, int nseg,
                                                            uint32_t tile0, InlineTable inl) {
    block_of_table<SegRec>(launch_table(table, inl), nseg, tile0, AccumTile<kOverwrite>{});
}

// ------------------------------------------------------------ merge delta

// merged = bf16 nearest-even of (f32(base) + delta): one binary32 addition.
struct MergeTile {
    __device__ __forceinline__ void operator()(const SegRec &r, uint32_t local_tile) const {
#pragma clang fp contract(off)
        const uint64_t base_w = r.p[0], delta = r.p[1], merged = r.p[2];
        const int64_t numel = r.numel;
        const int64_t base = int64_t(local_tile) * kTile;
        const int64_t lane = int64_t(threadIdx.x) * kVec;
        const bool vector_ok = base + kTile <= numel && ((base_w | merged) & 7) == 0 &&
                               (delta & 15) == 0;
        if (vector_ok) {
            u32x2 b2[kUnroll];
            f32x4 d4[kUnroll];
            const int vl = int(threadIdx.x);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;
                b2[u] = tile_ld<u32x2>(tile_rsrc<u32x2>(base_w, q0, kBlock), vl);
                d4[u] = tile_ld<f32x4>(tile_rsrc<f32x4>(delta, q0, kBlock), vl);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t q0 = (base + u * (kBlock * kVec)) / kVec;
                const float s0 = bf16_lo(b2[u].x) + d4[u].x, s1 = bf16_hi(b2[u].x) + d4[u].y;
                const float s2 = bf16_lo(b2[u].y) + d4[u].z, s3 = bf16_hi(b2[u].y) + d4[u].w;
                tile_st<u32x2>(tile_rsrc<u32x2>(merged, q0, kBlock), vl,
                               u32x2{to_bf16_pair(s0, s1), to_bf16_pair(s2, s3)});
            }
        } else {
            for (int u = 0; u < kUnroll; ++u) {
                for (int k = 0; k < kVec; ++k) {
                    const int64_t e = base + u * (kBlock * kVec) + lane + k;
                    if (e >= numel) continue;
                    const float sum = bf16_one(as_global<gu16>(base_w)[e]) + as_global<gfloat>(delta)[e];
                    as_global<gu16>(merged)[e] = to_bf16_one(sum);
                }
            }
        }
    }
};

__global__ __launch_bounds__(kBlock) void merge_tile_kernel(const void *table, int nseg,
                                                            uint32_t tile0, InlineTable inl) {
    block_of_table<SegRec>(launch_table(table, inl), nseg, tile0, MergeTile{});
}

// ------------------------------------------------- measurement aids

// Plain copy, one 16-byte vector per lane and one 256-lane workgroup per
// 4 KiB, with nontemporal loads and stores: the best plain-copy shape
// measured on MI355X, used as the practical read+write ceiling and as the
// known-size reference for HBM byte counters.
constexpr int kCopyBlock = 256;

__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const f32x4 *__restrict__ src,
                                                          f32x4 *__restrict__ dst, size_t n16,
                                                          size_t block0) {
    const size_t i = (block0 + blockIdx.x) * kCopyBlock + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Residency probe: the first wavefront of each workgroup notes its compute
// unit (XCC_ID and the HW_ID register) and the device wall clock, stays
// resident for `ticks` of that clock (a bounded wait), and notes the clock
// again.  The workgroup's LDS is whatever the launch reserves; the most
// workgroups that overlap in time on one compute unit is how many of them
// fit there.  rec holds 3 words per workgroup of the grid.
__global__ void residency_probe_kernel(uint64_t *__restrict__ rec, uint64_t ticks) {
    if (threadIdx.x != 0) return;
    constexpr int kHwIdReg = 4 | (31 << 11);      // hwreg(HW_REG_HW_ID, 0, 32)
    constexpr int kXccIdReg = 20 | (3 << 11);     // hwreg(HW_REG_XCC_ID, 0, 4)
    const uint32_t hw = __builtin_amdgcn_s_getreg(kHwIdReg);
    const uint32_t xcc = __builtin_amdgcn_s_getreg(kXccIdReg);
    const uint64_t t0 = wall_clock64();
    uint64_t t1 = t0;
    for (int i = 0; i < (1 << 22) && t1 - t0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(2);
        t1 = wall_clock64();
    }
    uint64_t *r = rec + 3 * uint64_t(blockIdx.x);
    r[0] = (uint64_t(xcc) << 32) | hw;
    r[1] = t0;
    r[2] = t1;
}

// The division, square root and bf16 rounding exactly as the AdamW kernel
// compiles them, for checking against IEEE results on the host.
__global__ __launch_bounds__(kBlock) void fp32_probe_kernel(const float *__restrict__ a,
                                                            const float *__restrict__ b,
                                                            float *__restrict__ quot,
                                                            float *__restrict__ root,
                                                            uint16_t *__restrict__ bf16,
                                                            int64_t n) {
#pragma clang fp contract(off)
    const int64_t stride = int64_t(gridDim.x) * kBlock;
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        quot[i] = a[i] / b[i];
        root[i] = __builtin_sqrtf(a[i]);
        bf16[i] = to_bf16_one(a[i]);
    }
}

}  // namespace

// Launches go through hipLaunchKernel, which returns the launch status
// directly instead of through the thread's sticky last-error slot.  Grids
// larger than max_blocks_per_launch are split into consecutive launches.
// The tile kernels always take an InlineTable argument; launches on a
// device table pass this unused one.
const InlineTable kNoInlineTable = {};
const void *adamw_kernel_fn(GradMode grad_mode, bool with_delta, int nmb) {
#define LEMA_PICK(M) with_delta ? reinterpret_cast<const void *>(&adamw_tile_kernel<M, true>) \
                                : reinterpret_cast<const void *>(&adamw_tile_kernel<M, false>)
    switch (grad_mode) {
    case kGradBf16: return LEMA_PICK(kGradBf16);
    case kGradF32: return LEMA_PICK(kGradF32);
    case kGradF32PlusBf16: return LEMA_PICK(kGradF32PlusBf16);
    case kGradBf16Sum:
        if (nmb < 1 || nmb > kMaxMicrobatches) return nullptr;
        return pick_sum_kernel(nmb, with_delta, std::make_index_sequence<kMaxMicrobatches>{});
    default: return nullptr;
    }
#undef LEMA_PICK
}

hipError_t launch_adamw(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, GradMode grad_mode, bool with_delta,
                        const AdamwConsts &c, hipStream_t stream, int nmb, uint32_t lds_bytes) {
    const void *fn = adamw_kernel_fn(grad_mode, with_delta, nmb);
    if (fn == nullptr || (table == nullptr) == (inl == nullptr)) return hipErrorInvalidValue;
    AdamwConsts consts = c;
    void *inl_arg = const_cast<InlineTable *>(inl ? inl : &kNoInlineTable);
    for (uint32_t tile0 = 0; tile0 < total_tiles;) {
        const uint32_t n = std::min<uint32_t>(total_tiles - tile0, max_blocks_per_launch(kBlock));
        void *args[] = {&table, &nseg, &tile0, &consts, inl_arg};
        hipError_t e = hipLaunchKernel(fn, dim3(n), dim3(kBlock), args, lds_bytes, stream);
        if (e != hipSuccess) return e;
        tile0 += n;
    }
    return hipSuccess;
}

hipError_t launch_accum(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, bool overwrite, hipStream_t stream) {
    if ((table == nullptr) == (inl == nullptr)) return hipErrorInvalidValue;
    const void *fn = overwrite ? reinterpret_cast<const void *>(&accum_tile_kernel<true>)
                               : reinterpret_cast<const void *>(&accum_tile_kernel<false>);
    void *inl_arg = const_cast<InlineTable *>(inl ? inl : &kNoInlineTable);
    for (uint32_t tile0 = 0; tile0 < total_tiles;) {
        const uint32_t n = std::min<uint32_t>(total_tiles - tile0, max_blocks_per_launch(kBlock));
        void *args[] = {&table, &nseg, &tile0, inl_arg};
        hipError_t e = hipLaunchKernel(fn, dim3(n), dim3(kBlock), args, 0, stream);
        if (e != hipSuccess) return e;
        tile0 += n;
    }
    return hipSuccess;
}

hipError_t launch_merge(const void *table, const InlineTable *inl, int nseg,
                        uint32_t total_tiles, hipStream_t stream) {
    if ((table == nullptr) == (inl == nullptr)) return hipErrorInvalidValue;
    void *inl_arg = const_cast<InlineTable *>(inl ? inl : &kNoInlineTable);
    for (uint32_t tile0 = 0; tile0 < total_tiles;) {
        const uint32_t n = std::min<uint32_t>(total_tiles - tile0, max_blocks_per_launch(kBlock));
        void *args[] = {&table, &nseg, &tile0, inl_arg};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&merge_tile_kernel), dim3(n),
                                       dim3(kBlock), args, 0, stream);
        if (e != hipSuccess) return e;
        tile0 += n;
    }
    return hipSuccess;
}

hipError_t launch_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const f32x4 *s = static_cast<const f32x4 *>(src);
    f32x4 *d = static_cast<f32x4 *>(dst);
    size_t n16 = bytes / 16;
    const size_t blocks = (n16 + kCopyBlock - 1) / kCopyBlock;
    for (size_t block0 = 0; block0 < blocks;) {
        const size_t n = std::min<size_t>(blocks - block0, max_blocks_per_launch(kCopyBlock));
        void *args[] = {&s, &d, &n16, &block0};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&copy_kernel),
                                       dim3(unsigned(n)), dim3(kCopyBlock), args, 0, stream);
        if (e != hipSuccess) return e;
        block0 += n;
    }
    return hipSuccess;
}

hipError_t launch_residency_probe(uint64_t *rec, int workgroups, int lanes, uint32_t lds_bytes,
                                  uint64_t ticks, hipStream_t stream) {
    void *args[] = {&rec, &ticks};
    return hipLaunchKernel(reinterpret_cast<const void *>(&residency_probe_kernel),
                           dim3(unsigned(workgroups)), dim3(unsigned(lanes)), args, lds_bytes,
                           stream);
}

hipError_t launch_fp32_probe(const float *a, const float *b, float *quot, float *root,
                             uint16_t *bf16, int64_t n, hipStream_t stream) {
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    void *args[] = {&a, &b, &quot, &root, &bf16, &n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&fp32_probe_kernel),
                           dim3(unsigned(blocks)), dim3(kBlock), args, 0, stream);
}

}  // namespace lema
