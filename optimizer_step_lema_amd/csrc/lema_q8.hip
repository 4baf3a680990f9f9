// lema_q8.hip -- gfx950 kernels of the int8 + per-row-scale path.
//
// LEMA README, "Quantization": with opt_state_bits = 8 and grad_acc_bits = 8
// Adam's moments and the gradient accumulators stay int8 with one scale per
// row and are dequantized only inside the per-layer AdamW step.  The storage
// (symmetric absmax scaling, 127 levels per sign) is stated in
// include/lema.h.
//
// Row teams.  The new codes of a row depend on the absmax of the whole new
// row, so each row belongs to one team of S lanes (S a power of two up to the
// workgroup size: 256 lanes, or 1024 for rows beyond 4096 elements) that keeps
// the row's new values in registers, at most 4 chunks per lane, until the
// team has reduced the absmax.  Chunk c of team lane l holds row elements
// 4*(c*S + l) .. 4*(c*S + l) + 3, so one chunk step of a team covers a
// contiguous run of 4*S elements: 16-byte fp32, 8-byte bf16 and 4-byte int8
// accesses, contiguous across the team.  Teams of at most 64 lanes lie inside
// one wavefront and reduce with cross-lane shuffles; wider teams add one LDS
// exchange behind a workgroup barrier (every lane reaches it: the team width
// is uniform across the workgroup, whose rows all come from one segment).
//
// Each lane issues all its loads before any arithmetic, since stores through
// the table's pointers could alias later loads as far as the compiler knows.
// The fp32 outputs of the step (master, bf16 weight, delta) are stored as
// soon as they are computed; the codes and scales follow the reduction.
//
// Arithmetic: the fp32 step of lema_kernels.hip element for element;
// dequantization is one binary32 multiplication f32(code) * scale;
// quantization divides by the scale with the IEEE division, rounds half to
// even (v_rndne_f32) and clamps to [-127, 127].  Absmax is taken on the
// magnitude bits as unsigned integers, so a NaN anywhere in a row dominates
// (giving a NaN scale) and the result does not depend on reduction order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lema_device.h"
#include "lema_internal.h"

namespace lema {
namespace {

using namespace dev;

typedef LEMA_GLOBAL int8_t gi8;
typedef LEMA_GLOBAL uint32_t gu32;

// ------------------------------------------------------------- codes

// The code in byte k of a packed word, widened exactly to fp32.
__device__ __forceinline__ float code_at(uint32_t word, int k) {
    return static_cast<float>(static_cast<int32_t>(word << (24 - 8 * k)) >> 24);
}

__device__ __forceinline__ float dequant(float code, float scale) {
#pragma clang fp contract(off)
    return code * scale;
}

// Magnitude bits: for non-NaN values their unsigned order is the order of
// |x|; every NaN lies above +inf.
__device__ __forceinline__ uint32_t mag_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// Scale of a row from its absmax bits: absmax / 127 (NaN stays NaN).
__device__ __forceinline__ float scale_of(uint32_t absmax_bits) {
#pragma clang fp contract(off)
    return __uint_as_float(absmax_bits) / 127.0f;
}

// Codes are only formed from a finite positive scale; other rows get zeros.
__device__ __forceinline__ bool usable(float scale) {
    return scale > 0.0f && mag_bits(scale) < 0x7F800000u;
}

__device__ __forceinline__ int32_t quant(float x, float scale) {
#pragma clang fp contract(off)
    float k = __builtin_rintf(x / scale);
    k = __builtin_fminf(__builtin_fmaxf(k, -127.0f), 127.0f);
    return static_cast<int32_t>(k);
}

__device__ __forceinline__ uint32_t pack4(int32_t a, int32_t b, int32_t c, int32_t d) {
    return (uint32_t(a) & 0xFFu) | ((uint32_t(b) & 0xFFu) << 8) | ((uint32_t(c) & 0xFFu) << 16) |
           (uint32_t(d) << 24);
}

// ---------------------------------------------------------- row teams

struct Team {
    int64_t row;     // row index within the segment
    int64_t first;   // element index of the row's first element
    int64_t len;     // elements of this row; 0 when the team has no row
    int lane;        // lane within the team
    int width;       // S
    int log2w;
    int chunks;
    bool vec;        // full chunks take vector accesses
};

template <int kThreads>
__device__ __forceinline__ Team team_of(const Q8Rec &r, uint32_t local_block) {
    Team t;
    t.log2w = r.team_log2;
    t.width = 1 << t.log2w;
    t.lane = int(threadIdx.x) & (t.width - 1);
    t.row = int64_t(local_block) * (kThreads >> t.log2w) + (int(threadIdx.x) >> t.log2w);
    t.first = t.row * r.row_len;
    t.len = t.row < r.rows ? std::min<int64_t>(r.row_len, r.numel - t.first) : 0;
    t.chunks = r.chunks;
    t.vec = (r.flags & kQVector) != 0;
    return t;
}

// Offset within the row of chunk c's first element.
__device__ __forceinline__ int64_t chunk_off(const Team &t, int c) {
    return 4 * (int64_t(c) * t.width + t.lane);
}

// Max over the team of two unsigned values.  Every lane of the workgroup
// must call it (it may contain a barrier).
template <int kThreads>
__device__ __forceinline__ void team_max2(const Team &t, uint32_t &a, uint32_t &b) {
    __shared__ uint32_t part[2][kThreads / 64];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        if (o < t.width) {
            a = std::max(a, uint32_t(__shfl_xor(int(a), o)));
            b = std::max(b, uint32_t(__shfl_xor(int(b), o)));
        }
    }
    if (t.width > 64) {
        const int wave = int(threadIdx.x) >> 6;
        if ((threadIdx.x & 63) == 0) {
            part[0][wave] = a;
            part[1][wave] = b;
        }
        __syncthreads();
        const int per_team = t.width >> 6;
        const int w0 = wave & ~(per_team - 1);
        for (int w = w0; w < w0 + per_team; ++w) {
            a = std::max(a, part[0][w]);
            b = std::max(b, part[1][w]);
        }
    }
}

// -------------------------------------------------------------- loads

// Four consecutive elements of one chunk.  Elements past the row's end read
// as zero (they are never stored and never enter an absmax).
__device__ __forceinline__ f32x4 load_f32(uint64_t base, int64_t e, bool full, bool vec,
                                          int64_t valid) {
    if (full && vec) return ld_nt<f32x4>(base, e >> 2);
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < 4; ++k)
        if (k < valid) x[k] = as_global<gfloat>(base)[e + k];
    return x;
}

__device__ __forceinline__ f32x4 load_bf16(uint64_t base, int64_t e, bool full, bool vec,
                                           int64_t valid) {
    if (full && vec) {
        const u32x2 p = ld_nt<u32x2>(base, e >> 2);
        return f32x4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
    }
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < 4; ++k)
        if (k < valid) x[k] = bf16_one(as_global<gu16>(base)[e + k]);
    return x;
}

// Four codes, packed as in memory (byte k = element k).
__device__ __forceinline__ uint32_t load_codes(uint64_t base, int64_t e, bool full, bool vec,
                                               int64_t valid) {
    if (full && vec) return ld_nt<uint32_t>(base, e >> 2);
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k)
        if (k < valid) w |= (uint32_t(uint8_t(as_global<gi8>(base)[e + k])) << (8 * k));
    return w;
}

__device__ __forceinline__ void store_f32(uint64_t base, int64_t e, bool full, bool vec,
                                          int64_t valid, f32x4 x) {
    if (full && vec) {
        st_nt<f32x4>(base, e >> 2, x);
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gfloat>(base)[e + k] = x[k];
}

__device__ __forceinline__ void store_bf16(uint64_t base, int64_t e, bool full, bool vec,
                                           int64_t valid, f32x4 x) {
    if (full && vec) {
        st_nt<u32x2>(base, e >> 2, u32x2{to_bf16_pair(x.x, x.y), to_bf16_pair(x.z, x.w)});
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gu16>(base)[e + k] = to_bf16_one(x[k]);
}

__device__ __forceinline__ void store_codes(uint64_t base, int64_t e, bool full, bool vec,
                                            int64_t valid, uint32_t w) {
    if (full && vec) {
        st_nt<uint32_t>(base, e >> 2, w);
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gi8>(base)[e + k] = int8_t(w >> (8 * k));
}

// Codes of four values against a row scale (all zero if it is not usable).
__device__ __forceinline__ uint32_t quant4(f32x4 x, float scale, bool ok) {
    if (!ok) return 0u;
    return pack4(quant(x.x, scale), quant(x.y, scale), quant(x.z, scale), quant(x.w, scale));
}

__device__ __forceinline__ uint32_t absmax4(uint32_t acc, f32x4 x, int64_t valid) {
    for (int k = 0; k < 4; ++k)
        if (k < valid) acc = std::max(acc, mag_bits(x[k]));
    return acc;
}

// ------------------------------------------------------------- AdamW

// One AdamW step with int8 moments (kMomQ8) and/or an int8 gradient
// accumulator (kGrad == kQGradQ8).  Record pointers:
//   {master, m, m_scale, v, v_scale, grad, grad_scale, weight, orig, delta}
template <bool kMomQ8, QGrad kGrad, bool kDelta, int kThreads>
struct AdamwRows {
    static constexpr int kMaxC = kQChunks;
    AdamwConsts c;

    __device__ __forceinline__ void operator()(const Q8Rec &r, uint32_t local_block) const {
        const uint64_t master = r.p[0], m = r.p[1], m_scale = r.p[2], v = r.p[3],
                       v_scale = r.p[4], grad = r.p[5], grad_scale = r.p[6], weight = r.p[7],
                       orig = r.p[8], delta = r.p[9];
        const Team t = team_of<kThreads>(r, local_block);
        const bool has_row = t.len > 0;
        const bool has_delta = kDelta && delta != 0;   // per segment within a delta launch

        float ms_old = 0.0f, vs_old = 0.0f, gs = 0.0f;
        if (has_row) {
            if constexpr (kMomQ8) {
                ms_old = as_global<gfloat>(m_scale)[t.row];
                vs_old = as_global<gfloat>(v_scale)[t.row];
            }
            if constexpr (kGrad == kQGradQ8) gs = as_global<gfloat>(grad_scale)[t.row];
        }

        // ---- loads of every chunk
        f32x4 w4[kMaxC], g4[kMaxC], mf[kMaxC], vf[kMaxC];
        uint32_t mc[kMaxC], vc[kMaxC], gc[kMaxC];
        u32x2 o2[kMaxC];
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            const int64_t e = t.first + off;
            const bool full = valid == 4;
            w4[ci] = load_f32(master, e, full, t.vec, valid);
            if constexpr (kMomQ8) {
                mc[ci] = load_codes(m, e, full, t.vec, valid);
                vc[ci] = load_codes(v, e, full, t.vec, valid);
            } else {
                mf[ci] = load_f32(m, e, full, t.vec, valid);
                vf[ci] = load_f32(v, e, full, t.vec, valid);
            }
            if constexpr (kGrad == kQGradBf16) g4[ci] = load_bf16(grad, e, full, t.vec, valid);
            if constexpr (kGrad == kQGradF32) g4[ci] = load_f32(grad, e, full, t.vec, valid);
            if constexpr (kGrad == kQGradQ8) gc[ci] = load_codes(grad, e, full, t.vec, valid);
            if (has_delta) {
                if (full && t.vec) {
                    o2[ci] = ld_nt<u32x2>(orig, e >> 2);
                } else {
                    uint32_t lo = 0, hi = 0;
                    for (int k = 0; k < 4; ++k) {
                        if (k >= valid) continue;
                        const uint32_t b = as_global<gu16>(orig)[e + k];
                        if (k < 2) lo |= b << (16 * k);
                        else hi |= b << (16 * (k - 2));
                    }
                    o2[ci] = u32x2{lo, hi};
                }
            }
        }

        // ---- the fp32 step; master, weight and delta go out at once
        uint32_t am = 0, av = 0;
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            const int64_t e = t.first + off;
            const bool full = valid == 4;
            f32x4 w = w4[ci], mm, vv, g;
            if constexpr (kMomQ8) {
                for (int k = 0; k < 4; ++k) {
                    mm[k] = dequant(code_at(mc[ci], k), ms_old);
                    vv[k] = dequant(code_at(vc[ci], k), vs_old);
                }
            } else {
                mm = mf[ci];
                vv = vf[ci];
            }
            if constexpr (kGrad == kQGradQ8) {
                for (int k = 0; k < 4; ++k) g[k] = dequant(code_at(gc[ci], k), gs);
            } else {
                g = g4[ci];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float wk = w[k], mk = mm[k], vk = vv[k];
                adamw_elem(wk, mk, vk, g[k], c);
                w[k] = wk;
                mm[k] = mk;
                vv[k] = vk;
            }
            store_f32(master, e, full, t.vec, valid, w);
            store_bf16(weight, e, full, t.vec, valid, w);
            if (has_delta) {
#pragma clang fp contract(off)
                const u32x2 o = o2[ci];
                const f32x4 d = {w.x - bf16_lo(o.x), w.y - bf16_hi(o.x), w.z - bf16_lo(o.y),
                                 w.w - bf16_hi(o.y)};
                store_f32(delta, e, full, t.vec, valid, d);
            }
            if constexpr (kMomQ8) {
                am = absmax4(am, mm, valid);
                av = absmax4(av, vv, valid);
                mf[ci] = mm;
                vf[ci] = vv;
            } else {
                store_f32(m, e, full, t.vec, valid, mm);
                store_f32(v, e, full, t.vec, valid, vv);
            }
        }
        if constexpr (!kMomQ8) return;

        // ---- requantize the moments against the new row scales
        team_max2<kThreads>(t, am, av);
        if (!has_row) return;
        const float ms = scale_of(am), vs = scale_of(av);
        const bool m_ok = usable(ms), v_ok = usable(vs);
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            const int64_t e = t.first + off;
            const bool full = valid == 4;
            store_codes(m, e, full, t.vec, valid, quant4(mf[ci], ms, m_ok));
            store_codes(v, e, full, t.vec, valid, quant4(vf[ci], vs, v_ok));
        }
        if (t.lane == 0) {
            as_global<gfloat>(m_scale)[t.row] = ms;
            as_global<gfloat>(v_scale)[t.row] = vs;
        }
    }
};

template <bool kMomQ8, QGrad kGrad, bool kDelta, int kThreads>
__global__ __launch_bounds__(kThreads) void adamw_q8_kernel(const void *table, int nseg,
                                                            uint32_t block0, AdamwConsts c) {
    block_of_table<Q8Rec>(table, nseg, block0, AdamwRows<kMomQ8, kGrad, kDelta, kThreads>{c});
}

// ------------------------------------------------------ accumulation

// int8 accumulator and one bf16 micro-batch: {codes, scale, grad_bf16}.
//   overwrite : acc = Q(f32(g))
//   otherwise : acc = Q(D(acc) + f32(g))
// The same team pattern serves the plain conversions of whole tensors:
// quantize {x, codes, scale} and dequantize (codes, scale -> x).
enum RowOp : int { kAccumAdd = 0, kAccumOverwrite = 1, kQuantize = 2, kDequantize = 3 };

template <RowOp kOp, int kThreads>
struct CodeRows {
    static constexpr int kMaxC = kQChunks;
    __device__ __forceinline__ void operator()(const Q8Rec &r, uint32_t local_block) const {
        const Team t = team_of<kThreads>(r, local_block);
        const bool has_row = t.len > 0;
        // pointers: accumulation {codes, scale, grad}; conversions {x, codes, scale}
        const uint64_t codes = (kOp == kAccumAdd || kOp == kAccumOverwrite) ? r.p[0] : r.p[1];
        const uint64_t scale = (kOp == kAccumAdd || kOp == kAccumOverwrite) ? r.p[1] : r.p[2];
        const uint64_t src = (kOp == kAccumAdd || kOp == kAccumOverwrite) ? r.p[2] : r.p[0];

        float s_old = 0.0f;
        if (has_row && (kOp == kAccumAdd || kOp == kDequantize))
            s_old = as_global<gfloat>(scale)[t.row];

        f32x4 x[kMaxC];
        uint32_t cw[kMaxC];
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            const int64_t e = t.first + off;
            const bool full = valid == 4;
            if constexpr (kOp == kAccumAdd || kOp == kDequantize)
                cw[ci] = load_codes(codes, e, full, t.vec, valid);
            if constexpr (kOp == kAccumAdd || kOp == kAccumOverwrite)
                x[ci] = load_bf16(src, e, full, t.vec, valid);
            if constexpr (kOp == kQuantize) x[ci] = load_f32(src, e, full, t.vec, valid);
        }

        uint32_t amax = 0, unused = 0;
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            if constexpr (kOp == kAccumAdd) {
                for (int k = 0; k < 4; ++k)
                    x[ci][k] = accum_elem(dequant(code_at(cw[ci], k), s_old), x[ci][k], false);
            }
            if constexpr (kOp == kDequantize) {
                f32x4 d;
                for (int k = 0; k < 4; ++k) d[k] = dequant(code_at(cw[ci], k), s_old);
                store_f32(src, t.first + off, valid == 4, t.vec, valid, d);
            } else {
                amax = absmax4(amax, x[ci], valid);
            }
        }
        if constexpr (kOp == kDequantize) return;

        team_max2<kThreads>(t, amax, unused);
        if (!has_row) return;
        const float s = scale_of(amax);
        const bool ok = usable(s);
#pragma unroll
        for (int ci = 0; ci < kMaxC; ++ci) {
            const int64_t off = chunk_off(t, ci);
            const int64_t valid = (ci < t.chunks) ? std::min<int64_t>(4, t.len - off) : 0;
            if (valid <= 0) continue;
            store_codes(codes, t.first + off, valid == 4, t.vec, valid, quant4(x[ci], s, ok));
        }
        if (t.lane == 0) as_global<gfloat>(scale)[t.row] = s;
    }
};

template <RowOp kOp, int kThreads>
__global__ __launch_bounds__(kThreads) void code_rows_kernel(const void *table, int nseg,
                                                             uint32_t block0) {
    block_of_table<Q8Rec>(table, nseg, block0, CodeRows<kOp, kThreads>{});
}

template <class... Args>
hipError_t launch_split(const void *fn, int block, uint32_t total_blocks, hipStream_t stream,
                        const void *table, int nseg, Args... extra) {
    for (uint32_t block0 = 0; block0 < total_blocks;) {
        const uint32_t n = std::min<uint32_t>(total_blocks - block0, kMaxBlocksPerLaunch);
        void *args[] = {&table, &nseg, &block0, &extra...};
        hipError_t e = hipLaunchKernel(fn, dim3(n), dim3(block), args, 0, stream);
        if (e != hipSuccess) return e;
        block0 += n;
    }
    return hipSuccess;
}

template <bool kMomQ8, QGrad kGrad, bool kDelta>
const void *pick_adamw(int block) {
    return block == kQBlock
               ? reinterpret_cast<const void *>(&adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlock>)
               : reinterpret_cast<const void *>(&adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlockWide>);
}

template <bool kMomQ8, QGrad kGrad>
const void *pick_adamw_delta(bool with_delta, int block) {
    return with_delta ? pick_adamw<kMomQ8, kGrad, true>(block)
                      : pick_adamw<kMomQ8, kGrad, false>(block);
}

template <RowOp kOp>
const void *pick_rows(int block) {
    return block == kQBlock ? reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlock>)
                            : reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlockWide>);
}

bool block_ok(int block) { return block == kQBlock || block == kQBlockWide; }

}  // namespace

hipError_t launch_adamw_q8(const void *table, int nseg, uint32_t total_blocks, bool moments_q8,
                           QGrad grad, bool with_delta, int block, const AdamwConsts &c,
                           hipStream_t stream) {
    if (!block_ok(block)) return hipErrorInvalidValue;
    const void *fn = nullptr;
    if (moments_q8) {
        switch (grad) {
        case kQGradBf16: fn = pick_adamw_delta<true, kQGradBf16>(with_delta, block); break;
        case kQGradF32: fn = pick_adamw_delta<true, kQGradF32>(with_delta, block); break;
        case kQGradQ8: fn = pick_adamw_delta<true, kQGradQ8>(with_delta, block); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        // fp32 moments only pair with an int8 gradient here; the other
        // combinations run on the tile kernels of lema_kernels.hip
        if (grad != kQGradQ8) return hipErrorInvalidValue;
        fn = pick_adamw_delta<false, kQGradQ8>(with_delta, block);
    }
    return launch_split(fn, block, total_blocks, stream, table, nseg, c);
}

hipError_t launch_accum_q8(const void *table, int nseg, uint32_t total_blocks, bool overwrite,
                           int block, hipStream_t stream) {
    if (!block_ok(block)) return hipErrorInvalidValue;
    const void *fn = overwrite ? pick_rows<kAccumOverwrite>(block) : pick_rows<kAccumAdd>(block);
    return launch_split(fn, block, total_blocks, stream, table, nseg);
}

hipError_t launch_quantize_q8(const void *table, int nseg, uint32_t total_blocks, bool dequantize,
                              int block, hipStream_t stream) {
    if (!block_ok(block)) return hipErrorInvalidValue;
    const void *fn = dequantize ? pick_rows<kDequantize>(block) : pick_rows<kQuantize>(block);
    return launch_split(fn, block, total_blocks, stream, table, nseg);
}

}  // namespace lema
