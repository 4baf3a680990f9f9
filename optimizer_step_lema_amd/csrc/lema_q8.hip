// lema_q8.hip -- gfx950 kernels of the int8 + per-row-scale path.
//
// LEMA README, "Quantization": 8-bit settings for the optimizer state and
// the gradient accumulator keep Adam's moments and the accumulators as int8
// codes with a scale per row, widened to fp32 only within the step.  The storage
// (symmetric absmax scaling, 127 levels per sign) is stated in
// include/lema.h.
//
// Row teams.  The new codes of a row depend on the absmax of the whole new
// row, so each row belongs to one team of S lanes (S a power of two up to the
// workgroup size: 256 lanes, or 1024 for the longest rows) that keeps the
// row's new values in registers until the team has reduced the absmax.
// Chunk c of team lane l holds row elements 4*(c*S + l) .. 4*(c*S + l) + 3,
// so one chunk step of a team covers a contiguous run of 4*S elements:
// 16-byte fp32, 8-byte bf16 and 4-byte int8 accesses, contiguous across the
// team.  Teams of at most 64 lanes lie inside one wavefront and reduce with
// DPP and row-swap instructions; wider teams add one LDS exchange behind a
// workgroup barrier (every lane reaches it: the team width is uniform across
// the workgroup, whose rows all come from one segment).
//
// Three kernel families share this mapping: wave rows (teams of whole
// wavefronts on aligned arrays, the common case: rows of about 500 to 16,384
// elements, every access through row-sized buffer resources), packed rows
// (rows of 4..256 elements, several rows per lane) and general row teams
// (everything else: misaligned arrays, short or odd rows, element-guarded
// accesses).
//
// Each lane issues all its loads before any arithmetic, since stores through
// the table's pointers could alias later loads as far as the compiler knows.
// The fp32 outputs of the step (master, bf16 weight, delta) are stored as
// soon as they are computed; the codes and scales follow the reduction.  In
// the general row teams, a lane whose chunks are all full vector chunks
// takes a path without per-chunk tests and other lanes the element-guarded
// one; the two paths meet before the team reduction, so its barrier is never
// inside a divergent branch.
//
// Arithmetic: the fp32 step of lema_kernels.hip element for element;
// dequantization is one binary32 multiplication f32(code) * scale;
// quantization gives the code of the IEEE quotient x / scale rounded half to
// even and clamped to [-127, 127], mostly without dividing (see QuantRow).
// Absmax is taken on the magnitude bits as unsigned integers, so a NaN
// anywhere in a row dominates (giving a NaN scale) and the result does not
// depend on reduction order.
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

// The per-row part of quantization.  Codes are formed only from a finite
// positive scale s (other rows get zeros).  When s is a normal number
// (s <= FLT_MAX/127, so 1/s is normal too), a reciprocal r with
// |r*s - 1| <= 2^-23 lets y = x*r serve in place of x/s:
//   |x| <= absmax and s >= absmax/127 (1 - 2^-24) bound |x/s| by 127.00002;
//   |y - x/s| <= |x/s| 2^-23 (r) + |x*r| 2^-24 (the product's rounding)
//   < 2.3e-5, and the IEEE quotient q = RN(x/s) is within 2^-18 of x/s;
//   so |y - q| < 2.7e-5 < 2^-15.
// So when y lies more than 2^-15 from the nearest half-integer, y and q lie
// strictly between the same two half-integers and round to the same integer,
// which is within [-127, 127].  The lane rounds y by adding 1.5 * 2^23: the
// sum is rounded to an integer, half to even, and its low byte is that
// integer's two's-complement byte.  A lane holding any value nearer to a
// half-integer (about 6e-5 of all values), and every lane of a row with a
// subnormal scale, takes the codes from the IEEE division instead.
//
// r is one Newton step from the hardware reciprocal r0 = 1/s (1 + d):
// e = fma(-s, r0, 1) = -d exactly rounded, r = fma(e, r0, r0) =
// RN(1/s (1 - d^2 - d e')), so |r*s - 1| <= 2^-24 + d^2 + 2^-24 |d|, inside
// 2^-23 for any |d| <= 2^-21, far more than v_rcp_f32's documented 1 ulp.
struct QuantRow {
    float s;      // the row's new scale
    float r;      // about 1/s (see above) when `fast`
    bool ok;      // codes are formed (else all zero)
    bool fast;    // s is normal: x*r decides away from half-integers
};

// The reciprocal of a normal scale s (see above).
__device__ __forceinline__ float row_reciprocal(float s) {
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

__device__ __forceinline__ QuantRow quant_row(uint32_t absmax_bits) {
#pragma clang fp contract(off)
    QuantRow q;
    q.s = scale_of(absmax_bits);
    q.ok = q.s > 0.0f && mag_bits(q.s) < 0x7F800000u;
    q.fast = q.ok && mag_bits(q.s) >= 0x00800000u;
    const float r = row_reciprocal(q.s);
    q.r = q.fast ? r : 0.0f;
    return q;
}

constexpr float kRoundMagic = 12582912.0f;    // 1.5 * 2^23
// y is decided by x*r when |y - round(y)| <= 1/2 - 2^-15 (see QuantRow)
constexpr float kFarFromHalf = 0.5f - 0x1p-15f;

// Packed codes of four values from y = x*r; `dmax` keeps the largest
// distance |y - round(y)| seen.  The codes are the low bytes of the rounded
// sums, gathered by byte permutes.
__device__ __forceinline__ uint32_t quant4_fast(f32x4 x, float r, float &dmax) {
#pragma clang fp contract(off)
    uint32_t g[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float y = x[k] * r;
        const float sum = y + kRoundMagic;      // integer nearest y, ties to even
        const float yk = sum - kRoundMagic;     // that integer, exactly
        dmax = __builtin_fmaxf(dmax, __builtin_fabsf(y - yk));
        g[k] = __float_as_uint(sum);
    }
    // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7
    // of the first, 12 gives zero
    const uint32_t lo = __builtin_amdgcn_perm(g[1], g[0], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(g[3], g[2], 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Packed codes of four values from the IEEE quotient x / s.
__device__ __forceinline__ uint32_t quant4_exact(f32x4 x, float s) {
#pragma clang fp contract(off)
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float q = __builtin_rintf(x[k] / s);
        q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
        w |= (uint32_t(static_cast<int32_t>(q)) & 0xFFu) << (8 * k);
    }
    return w;
}

__device__ __forceinline__ uint32_t absmax4(uint32_t acc, f32x4 x, int64_t valid) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (k < valid) acc = std::max(acc, mag_bits(x[k]));
    return acc;
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
    bool full;       // every chunk of this lane is a full vector chunk
};

// Offset within the row of chunk c's first element.
__device__ __forceinline__ int64_t chunk_off(const Team &t, int c) {
    return 4 * (int64_t(c) * t.width + t.lane);
}

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
    t.full = t.vec && t.len > 0 && chunk_off(t, t.chunks - 1) + 4 <= t.len;
    return t;
}

// Elements of chunk c inside the row (0 .. 4).
template <bool kFull>
__device__ __forceinline__ int64_t valid_of(const Team &t, int c) {
    if (c >= t.chunks) return 0;
    if constexpr (kFull) return 4;
    const int64_t rem = t.len - chunk_off(t, c);
    return rem <= 0 ? 0 : (rem < 4 ? rem : 4);
}

// Max over aligned groups of `width` lanes (a power of two; 64 and more
// mean the whole wavefront): every lane ends with its group's max.  Each
// level combines two neighbouring groups of the level before: quad
// permutations [1,0,3,2] and [2,3,0,1] for pairs and quads, the half-row and
// row mirrors (lane i reads lane 7-i, or 15-i, within 8 or 16) for 8 and 16,
// and the gfx950 row swaps (v_permlane16_swap, v_permlane32_swap: the two
// results hold a lane's own value and its partner's 16 or 32 lanes away)
// for 32 and 64.  `width` is the same on every lane, and every lane of the
// wavefront must be active.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_max(uint32_t a) {
    return std::max(a, uint32_t(__builtin_amdgcn_update_dpp(0, int(a), kCtrl, 0xF, 0xF, false)));
}

__device__ __forceinline__ uint32_t group_max(uint32_t a, int width) {
    if (width > 1) a = dpp_max<0xB1>(a);      // quad_perm [1,0,3,2]
    if (width > 2) a = dpp_max<0x4E>(a);      // quad_perm [2,3,0,1]
    if (width > 4) a = dpp_max<0x141>(a);     // row_half_mirror
    if (width > 8) a = dpp_max<0x140>(a);     // row_mirror
    if (width > 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(a, a, false, false);
        a = std::max(uint32_t(p[0]), uint32_t(p[1]));
    }
    if (width > 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(a, a, false, false);
        a = std::max(uint32_t(p[0]), uint32_t(p[1]));
    }
    return a;
}

// Max over the team of two unsigned values.  Every lane of the workgroup
// must call it (it may contain a barrier).
template <int kThreads>
__device__ __forceinline__ void team_max2(const Team &t, uint32_t &a, uint32_t &b) {
    __shared__ uint32_t part[2][kThreads / 64];
    a = group_max(a, t.width);
    b = group_max(b, t.width);
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

// -------------------------------------------------------------- access

// Four consecutive elements of one chunk: a vector access, or `valid`
// element accesses (elements past the row's end read as zero; they are never
// stored and never enter an absmax).
__device__ __forceinline__ f32x4 load_f32(uint64_t base, int64_t e, bool vector, int64_t valid) {
    if (vector) return ld_nt<f32x4>(base, e >> 2);
    f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < 4; ++k)
        if (k < valid) x[k] = as_global<gfloat>(base)[e + k];
    return x;
}

// bf16 bits of four elements, packed two per word.
__device__ __forceinline__ u32x2 load_bf16_bits(uint64_t base, int64_t e, bool vector,
                                                int64_t valid) {
    if (vector) return ld_nt<u32x2>(base, e >> 2);
    uint32_t h[4] = {0, 0, 0, 0};
    for (int k = 0; k < 4; ++k)
        if (k < valid) h[k] = as_global<gu16>(base)[e + k];
    return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

__device__ __forceinline__ f32x4 widen_bf16(u32x2 p) {
    return f32x4{bf16_lo(p.x), bf16_hi(p.x), bf16_lo(p.y), bf16_hi(p.y)};
}

// Four codes, packed as in memory (byte k = element k).
__device__ __forceinline__ uint32_t load_codes(uint64_t base, int64_t e, bool vector,
                                               int64_t valid) {
    if (vector) return ld_nt<uint32_t>(base, e >> 2);
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k)
        if (k < valid) w |= (uint32_t(uint8_t(as_global<gi8>(base)[e + k])) << (8 * k));
    return w;
}

__device__ __forceinline__ void store_f32(uint64_t base, int64_t e, bool vector, int64_t valid,
                                          f32x4 x) {
    if (vector) {
        st_nt<f32x4>(base, e >> 2, x);
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gfloat>(base)[e + k] = x[k];
}

__device__ __forceinline__ void store_bf16(uint64_t base, int64_t e, bool vector, int64_t valid,
                                           f32x4 x) {
    if (vector) {
        st_nt<u32x2>(base, e >> 2, u32x2{to_bf16_pair(x.x, x.y), to_bf16_pair(x.z, x.w)});
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gu16>(base)[e + k] = to_bf16_one(x[k]);
}

__device__ __forceinline__ void store_codes(uint64_t base, int64_t e, bool vector, int64_t valid,
                                            uint32_t w) {
    if (vector) {
        st_nt<uint32_t>(base, e >> 2, w);
        return;
    }
    for (int k = 0; k < 4; ++k)
        if (k < valid) as_global<gi8>(base)[e + k] = int8_t(w >> (8 * k));
}

// Quantize this lane's chunks of one row and store the codes.
template <int kC, bool kFull>
__device__ __forceinline__ void quantize_store(const Team &t, uint64_t codes, const QuantRow &q,
                                               const f32x4 (&x)[kC]) {
    uint32_t w[kC];
#pragma unroll
    for (int ci = 0; ci < kC; ++ci) w[ci] = 0;
    if (q.ok) {
        float dmax = 0.0f;
        if (q.fast) {
#pragma unroll
            for (int ci = 0; ci < kC; ++ci)
                if (valid_of<kFull>(t, ci) > 0) w[ci] = quant4_fast(x[ci], q.r, dmax);
        }
        if (!q.fast || dmax > kFarFromHalf) {
#pragma unroll
            for (int ci = 0; ci < kC; ++ci)
                if (valid_of<kFull>(t, ci) > 0) w[ci] = quant4_exact(x[ci], q.s);
        }
    }
#pragma unroll
    for (int ci = 0; ci < kC; ++ci) {
        const int64_t valid = valid_of<kFull>(t, ci);
        if (valid <= 0) continue;
        store_codes(codes, t.first + chunk_off(t, ci), kFull || (t.vec && valid == 4), valid,
                    w[ci]);
    }
}

// ------------------------------------------------------- packed rows
//
// Rows of 4*S elements, S a power of two of at most 64 lanes, are packed
// (kQPacked): a team of S lanes covers a whole row in one chunk step, so lane
// t's chunk c holds elements 4*(t mod S) .. +3 of row  row0 + c*G + t/S
// (G = kThreads/S teams per chunk step), and each chunk step of a wavefront
// is one contiguous run of 256 elements.  With the mapping above such rows
// would give a lane whole rows, and a wavefront's accesses would be strided
// by the row length.  Teams lie inside one wavefront, so the absmax
// reductions are shuffles only; each chunk belongs to its own row and scale.
struct Packed {
    int64_t row0;    // row of chunk 0
    int G;           // rows per chunk step
    int lane;        // lane within the team
    int width;       // S
};

template <int kThreads, int kC>
__device__ __forceinline__ Packed packed_of(const Q8Rec &r, uint32_t local_block) {
    Packed p;
    p.width = 1 << r.team_log2;
    p.G = kThreads >> r.team_log2;
    p.lane = int(threadIdx.x) & (p.width - 1);
    p.row0 = int64_t(local_block) * (int64_t(kC) * p.G) + (int(threadIdx.x) >> r.team_log2);
    return p;
}

// Chunk c of a packed lane: its row, first element and valid elements.
struct PackedChunk {
    int64_t row;
    int64_t e;
    int64_t valid;   // 0 .. 4
    bool has_row;
};

__device__ __forceinline__ PackedChunk packed_chunk(const Packed &p, const Q8Rec &r, int c) {
    PackedChunk k;
    k.row = p.row0 + int64_t(c) * p.G;
    const int64_t first = k.row * r.row_len;
    const int64_t len = k.row < r.rows ? std::min<int64_t>(r.row_len, r.numel - first) : 0;
    k.has_row = len > 0;
    k.e = first + 4 * int64_t(p.lane);
    const int64_t rem = len - 4 * int64_t(p.lane);
    k.valid = rem <= 0 ? 0 : (rem < 4 ? rem : 4);
    return k;
}


// Codes of one chunk against its row's quantization.
__device__ __forceinline__ uint32_t quant_chunk(const QuantRow &q, f32x4 x) {
    uint32_t w = 0;
    if (q.ok) {
        float dmax = 0.0f;
        if (q.fast) w = quant4_fast(x, q.r, dmax);
        if (!q.fast || dmax > kFarFromHalf) w = quant4_exact(x, q.s);
    }
    return w;
}

// --------------------------------------------------------- wave rows
//
// Rows whose team spans whole wavefronts (S >= 64 lanes), on vector-aligned
// arrays whose element count is a multiple of 4 (kQWave), run in kernels of
// their own.  Every lane of a wavefront works on the same row, so the row,
// its first element and its length are wave-uniform and sit in scalar
// registers; each array is reached through a buffer resource based at the
// row's first element and sized to the row, and chunk c of team lane l is
// vector c*S + l of that resource.  No per-chunk 64-bit address arithmetic
// is left.  A chunk lies wholly inside the row or wholly past its end (the
// length is a multiple of 4): the resource's range check reads the latter
// as zeros and drops its stores, and the lane leaves it out of the absmax.
// A team without a row (past the segment's last row) has a zero-sized
// resource and only takes part in the team reduction.
struct WaveRow {
    int64_t row;     // row index within the segment (wave-uniform)
    int64_t first;   // element index of the row's first element
    int32_t len;     // elements of the row; 0 when the team has no row
    int32_t nvec;    // len / 4
    int32_t lane;    // lane within the team
    int32_t width;   // S
    int32_t chunks;  // chunks per lane of the segment's rows
};

template <int kThreads>
__device__ __forceinline__ WaveRow wave_row_of(const Q8Rec &r, uint32_t local_block) {
    WaveRow w;
    const int log2w = r.team_log2;    // at least 6
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    w.width = 1 << log2w;
    w.lane = int(threadIdx.x) & (w.width - 1);
    w.row = int64_t(local_block) * (kThreads >> log2w) + (wave >> (log2w - 6));
    w.first = w.row * r.row_len;
    w.len = w.row < r.rows ? int32_t(std::min<int64_t>(r.row_len, r.numel - w.first)) : 0;
    w.nvec = w.len >> 2;
    w.chunks = r.chunks;
    return w;
}

// The buffer resource of one array (kBytes per element) over the row.
template <int kBytes>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(uint64_t array, const WaveRow &w) {
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(array + uint64_t(w.first) * kBytes), 0, w.len * kBytes,
        kRawBufferWord3);
}

// Vector v (elements 4v .. 4v+3) of a row's array.  Accesses are
// nontemporal (gfx950 NT bit), like the global accesses of the other int8
// paths, except the reads of the one-byte code arrays in the separate
// wave-row launches (the step's m and v codes, an int8 gradient, the
// accumulator), which take the default policy.  Measured on MI355X with
// variant builds, interleaved on one box, state rotated so that no code
// array fits the last-level cache between its uses: the int8 step over the
// Llama-2-7B attention projections went from 1.004-1.011 to 0.965-0.975 ms
// (two boxes), eight int8 accumulations of one layer, each behind a 2 GiB
// cache scrub, from 1.091 to 1.048-1.050 ms, the whole 7B step stayed at
// 23.8-24.0 ms; in the mixed launch the rank-16 LoRA step lost 2% with it
// (0.171-0.174 against 0.174-0.177 ms), and default-policy code writes or
// fp32 reads gained nothing anywhere (every array on the default policy
// took the attention step to 1.094-1.099 ms).
constexpr int kRowPolicy = 2;
constexpr int kCodeLoadPolicy = 0;

template <int kPolicy>
__device__ __forceinline__ uint32_t row_ld_codes(__amdgpu_buffer_rsrc_t r, uint32_t v) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, int(v * 4), 0, kPolicy);
}
__device__ __forceinline__ u32x2 row_ld_bf16(__amdgpu_buffer_rsrc_t r, uint32_t v) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, int(v * 8), 0, kRowPolicy));
}
__device__ __forceinline__ f32x4 row_ld_f32(__amdgpu_buffer_rsrc_t r, uint32_t v) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(v * 16), 0, kRowPolicy));
}
__device__ __forceinline__ void row_st_codes(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t w) {
    __builtin_amdgcn_raw_buffer_store_b32(w, r, int(v * 4), 0, kRowPolicy);
}
__device__ __forceinline__ void row_st_bf16(__amdgpu_buffer_rsrc_t r, uint32_t v, f32x4 x) {
    const u32x2_t b = {to_bf16_pair(x.x, x.y), to_bf16_pair(x.z, x.w)};
    __builtin_amdgcn_raw_buffer_store_b64(b, r, int(v * 8), 0, kRowPolicy);
}
__device__ __forceinline__ void row_st_f32(__amdgpu_buffer_rsrc_t r, uint32_t v, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, int(v * 16), 0,
                                           kRowPolicy);
}

// Max over a wave-rows team of kN values: the wavefront's reduction, then,
// for teams of several wavefronts, one LDS exchange behind a workgroup
// barrier that every lane reaches (the team width is the same across the
// workgroup).
template <int kThreads, int kN>
__device__ __forceinline__ void wave_team_max(uint32_t (&a)[kN], int width) {
#pragma unroll
    for (int i = 0; i < kN; ++i) a[i] = group_max(a[i], 64);
    if constexpr (kThreads > 64) {
        __shared__ uint32_t part[kN][kThreads / 64];
        if (width > 64) {
            const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
            if ((threadIdx.x & 63) == 0) {
#pragma unroll
                for (int i = 0; i < kN; ++i) part[i][wave] = a[i];
            }
            __syncthreads();
            const int per_team = width >> 6;
            const int w0 = wave & ~(per_team - 1);
            for (int k = 0; k < per_team; ++k) {
#pragma unroll
                for (int i = 0; i < kN; ++i) a[i] = std::max(a[i], part[i][w0 + k]);
            }
        }
    }
}

// Codes of a lane's first `chunks` chunks against its row's quantization
// (the words past `chunks` are left unset: no caller reads them).
template <int kC>
__device__ __forceinline__ void quant_lane(const QuantRow &q, const f32x4 (&x)[kC], int chunks,
                                           uint32_t (&w)[kC]) {
    if (!q.ok) {
#pragma unroll
        for (int c = 0; c < kC; ++c)
            if (c < chunks) w[c] = 0;
        return;
    }
    float dmax = 0.0f;
    if (q.fast) {
#pragma unroll
        for (int c = 0; c < kC; ++c)
            if (c < chunks) w[c] = quant4_fast(x[c], q.r, dmax);
    }
    if (!q.fast || dmax > kFarFromHalf) {
#pragma unroll
        for (int c = 0; c < kC; ++c)
            if (c < chunks) w[c] = quant4_exact(x[c], q.s);
    }
}

// int8 codes of a wave-rows team through LDS: each wavefront moves the codes
// of 4 chunks (4 spans of 256 elements, one per chunk) as one 16-byte access
// per lane instead of four 4-byte ones, and LDS turns the spans around between
// that layout (lane j holds 16 codes of span j/16) and the chunk layout of the
// fp32 arrays (lane t holds 4 codes of every span).  A wavefront's code
// accesses are then 1 KB each, like its fp32 accesses; with 4-byte code
// accesses the step issued as many vector memory instructions per element as
// the fp32 step while moving two thirds of the bytes, and the address FIFO
// in front of the texture unit was full about a quarter of the time.
// One buffer per workgroup: kGroups groups of 4 chunks, for m and for v, per
// wavefront (1 KB each).
template <int kThreads, int kGroups>
__device__ __forceinline__ uint32_t *code_stage() {
    __shared__ __attribute__((aligned(16))) uint32_t buf[kThreads / 64][2][kGroups][256];
    return &buf[0][0][0][0];
}

// ------------------------------------------------------------- AdamW

// One AdamW step with int8 moments (kMomQ8) and/or an int8 gradient
// accumulator (kGrad == kQGradQ8).  Record pointers:
//   {master, m, m_scale, v, v_scale, grad, grad_scale, weight, orig, delta}
template <bool kMomQ8, QGrad kGrad, bool kDelta, int kThreads, int kRows>
struct AdamwRows {
    static constexpr int kC = kThreads == kQBlockWide ? kQWideChunks : kQStepChunks;
    AdamwConsts c;

    struct Row {
        uint64_t master, m, m_scale, v, v_scale, grad, grad_scale, weight, orig, delta;
        bool has_delta;
        float ms, vs, gs;    // old row scales (int8 arrays only)
    };

    // One chunk's inputs, as loaded.
    struct ChunkIn {
        f32x4 w, mf, vf, g4;
        uint32_t mc, vc, gc;
        u32x2 gb, o2;
    };

    __device__ __forceinline__ void load_chunk(const Row &R, int64_t e, bool vector,
                                               int64_t valid, ChunkIn &in) const {
        in.w = load_f32(R.master, e, vector, valid);
        if constexpr (kMomQ8) {
            in.mc = load_codes(R.m, e, vector, valid);
            in.vc = load_codes(R.v, e, vector, valid);
        } else {
            in.mf = load_f32(R.m, e, vector, valid);
            in.vf = load_f32(R.v, e, vector, valid);
        }
        if constexpr (kGrad == kQGradBf16) in.gb = load_bf16_bits(R.grad, e, vector, valid);
        if constexpr (kGrad == kQGradF32) in.g4 = load_f32(R.grad, e, vector, valid);
        if constexpr (kGrad == kQGradQ8) in.gc = load_codes(R.grad, e, vector, valid);
        if (R.has_delta) in.o2 = load_bf16_bits(R.orig, e, vector, valid);
    }

    // The fp32 step of one chunk with its row's old scales: the new master
    // weight w, moments mm, vv and (with delta) the delta d.
    __device__ __forceinline__ void step_math(const ChunkIn &in, bool has_delta, float ms,
                                              float vs, float gs, f32x4 &w, f32x4 &mm,
                                              f32x4 &vv, f32x4 &d) const {
        f32x4 g;
        w = in.w;
        if constexpr (kMomQ8) {
            for (int k = 0; k < 4; ++k) {
                mm[k] = dequant(code_at(in.mc, k), ms);
                vv[k] = dequant(code_at(in.vc, k), vs);
            }
        } else {
            mm = in.mf;
            vv = in.vf;
        }
        if constexpr (kGrad == kQGradQ8) {
            for (int k = 0; k < 4; ++k) g[k] = dequant(code_at(in.gc, k), gs);
        } else if constexpr (kGrad == kQGradBf16) {
            g = widen_bf16(in.gb);
        } else {
            g = in.g4;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float wk = w[k], mk = mm[k], vk = vv[k];
            adamw_elem(wk, mk, vk, g[k], c);
            w[k] = wk;
            mm[k] = mk;
            vv[k] = vk;
        }
        if (has_delta) {
#pragma clang fp contract(off)
            const f32x4 o = widen_bf16(in.o2);
            d = f32x4{w.x - o.x, w.y - o.y, w.z - o.z, w.w - o.w};
        }
    }

    // step_math, then the stores of master, weight, delta (and of fp32
    // moments); int8 moments come back in mm, vv.
    __device__ __forceinline__ void step_chunk(const Row &R, int64_t e, bool vector,
                                               int64_t valid, const ChunkIn &in, float ms,
                                               float vs, float gs, f32x4 &mm,
                                               f32x4 &vv) const {
        f32x4 w, d;
        step_math(in, R.has_delta, ms, vs, gs, w, mm, vv, d);
        store_f32(R.master, e, vector, valid, w);
        store_bf16(R.weight, e, vector, valid, w);
        if (R.has_delta) store_f32(R.delta, e, vector, valid, d);
        if constexpr (!kMomQ8) {
            store_f32(R.m, e, vector, valid, mm);
            store_f32(R.v, e, vector, valid, vv);
        }
    }

    // Loads, the fp32 step and the stores of master, weight, delta (and of
    // fp32 moments); int8 moments are left in mf/vf with their absmax bits.
    template <bool kFull>
    __device__ __forceinline__ void step_lane(const Team &t, const Row &R, f32x4 (&mf)[kC],
                                              f32x4 (&vf)[kC], uint32_t &am,
                                              uint32_t &av) const {
        ChunkIn in[kC];
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            const int64_t valid = valid_of<kFull>(t, ci);
            if (valid <= 0) continue;
            load_chunk(R, t.first + chunk_off(t, ci), kFull || (t.vec && valid == 4), valid, in[ci]);
        }

#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            const int64_t valid = valid_of<kFull>(t, ci);
            if (valid <= 0) continue;
            f32x4 mm, vv;
            step_chunk(R, t.first + chunk_off(t, ci), kFull || (t.vec && valid == 4), valid, in[ci],
                       R.ms, R.vs, R.gs, mm, vv);
            if constexpr (kMomQ8) {
                am = absmax4(am, mm, valid);
                av = absmax4(av, vv, valid);
                mf[ci] = mm;
                vf[ci] = vv;
            }
        }
    }

    // Packed rows: each chunk is a row of its own (see Packed).
    __device__ __forceinline__ void packed_rows(const Q8Rec &r, uint32_t local_block) const {
        const Row R{r.p[0], r.p[1], r.p[2], r.p[3], r.p[4], r.p[5], r.p[6], r.p[7], r.p[8],
                    r.p[9], kDelta && r.p[9] != 0, 0.0f, 0.0f, 0.0f};
        const Packed p = packed_of<kThreads, kC>(r, local_block);
        PackedChunk k[kC];
        ChunkIn in[kC];
        float ms[kC], vs[kC], gs[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            k[c] = packed_chunk(p, r, c);
            ms[c] = vs[c] = gs[c] = 0.0f;
            if (k[c].has_row) {
                if constexpr (kMomQ8) {
                    ms[c] = as_global<gfloat>(R.m_scale)[k[c].row];
                    vs[c] = as_global<gfloat>(R.v_scale)[k[c].row];
                }
                if constexpr (kGrad == kQGradQ8) gs[c] = as_global<gfloat>(R.grad_scale)[k[c].row];
            }
            if (k[c].valid > 0) load_chunk(R, k[c].e, k[c].valid == 4, k[c].valid, in[c]);
        }
        f32x4 mf[kC], vf[kC];
        uint32_t am[kC], av[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            am[c] = av[c] = 0;
            if (k[c].valid <= 0) continue;
            step_chunk(R, k[c].e, k[c].valid == 4, k[c].valid, in[c], ms[c], vs[c], gs[c],
                       mf[c], vf[c]);
            if constexpr (kMomQ8) {
                am[c] = absmax4(0u, mf[c], k[c].valid);
                av[c] = absmax4(0u, vf[c], k[c].valid);
            }
        }
        if constexpr (!kMomQ8) return;
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            am[c] = group_max(am[c], p.width);
            av[c] = group_max(av[c], p.width);
        }
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            if (!k[c].has_row) continue;
            const QuantRow qm = quant_row(am[c]), qv = quant_row(av[c]);
            if (k[c].valid > 0) {
                store_codes(R.m, k[c].e, k[c].valid == 4, k[c].valid, quant_chunk(qm, mf[c]));
                store_codes(R.v, k[c].e, k[c].valid == 4, k[c].valid, quant_chunk(qv, vf[c]));
            }
            if (p.lane == 0) {
                as_global<gfloat>(R.m_scale)[k[c].row] = qm.s;
                as_global<gfloat>(R.v_scale)[k[c].row] = qv.s;
            }
        }
    }

    // Wave rows (see WaveRow), with up to kCW chunks per lane.
    template <int kCW>
    __device__ __forceinline__ void wave_rows(const Q8Rec &r, uint32_t local_block) const {
        constexpr int kMomBytes = kMomQ8 ? 1 : 4;
        constexpr int kGradBytes = kGrad == kQGradBf16 ? 2 : kGrad == kQGradF32 ? 4 : 1;
        // code reads: the default policy in the separate wave-row launches,
        // nontemporal in the mixed one (see row_ld_codes)
        constexpr int kCodePolicy = kRows == kQRowsMixed ? kRowPolicy : kCodeLoadPolicy;
        const WaveRow wr = wave_row_of<kThreads>(r, local_block);
        const bool has_delta = kDelta && r.p[9] != 0;
        const auto r_master = row_rsrc<4>(r.p[0], wr);
        const auto r_m = row_rsrc<kMomBytes>(r.p[1], wr);
        const auto r_v = row_rsrc<kMomBytes>(r.p[3], wr);
        const auto r_g = row_rsrc<kGradBytes>(r.p[5], wr);
        const auto r_w = row_rsrc<2>(r.p[7], wr);
        const auto r_o = row_rsrc<2>(r.p[8], wr);
        const auto r_d = row_rsrc<4>(r.p[9], wr);
        float ms = 0.0f, vs = 0.0f, gs = 0.0f;
        if (wr.len > 0) {
            if constexpr (kMomQ8) {
                ms = as_global<gfloat>(r.p[2])[wr.row];
                vs = as_global<gfloat>(r.p[4])[wr.row];
            }
            if constexpr (kGrad == kQGradQ8) gs = as_global<gfloat>(r.p[6])[wr.row];
        }

        // 16-byte code accesses: rows (all of the segment's, and this one) of
        // a multiple of 16 elements in code arrays aligned to 16 bytes (the
        // test is uniform over the team)
        constexpr int kG = (kCW + 3) / 4;
        constexpr int kStageGroups =
            kRows == kQRowsMixed ? (kQMixedWaveChunks + 3) / 4 : (kC + 3) / 4;
        static_assert(kG <= kStageGroups, "code staging groups");
        const bool wide = kMomQ8 && (wr.len & 15) == 0 && (r.row_len & 15) == 0 &&
                          ((r.p[1] | r.p[3]) & 15) == 0;
        const int j = int(threadIdx.x) & 63;           // lane in the wavefront
        const int wt = wr.lane >> 6;                    // wavefront in the team
        uint32_t *stage = code_stage<kThreads, kStageGroups>() +
                          (int(threadIdx.x) >> 6) * (2 * kStageGroups * 256);
        // byte offset of lane j's 16 codes of group g: span 4g + j/16, part j % 16
        auto wide_off = [&](int g) {
            return ((4 * g + (j >> 4)) * wr.width + 64 * wt + (j & 15) * 4) * 4;
        };

        ChunkIn in[kCW];
        if (wide) {
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                if (4 * g + (j >> 4) >= wr.chunks) continue;
                const u32x4_t qm = __builtin_amdgcn_raw_buffer_load_b128(r_m, wide_off(g), 0, kCodePolicy);
                const u32x4_t qv = __builtin_amdgcn_raw_buffer_load_b128(r_v, wide_off(g), 0, kCodePolicy);
                *reinterpret_cast<u32x4_t *>(stage + g * 256 + 4 * j) = qm;
                *reinterpret_cast<u32x4_t *>(stage + (kStageGroups + g) * 256 + 4 * j) = qv;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int ci = 0; ci < kCW; ++ci) {
                if (ci >= wr.chunks) continue;
                in[ci].mc = stage[(ci >> 2) * 256 + (ci & 3) * 64 + j];
                in[ci].vc = stage[(kStageGroups + (ci >> 2)) * 256 + (ci & 3) * 64 + j];
            }
        }
#pragma unroll
        for (int ci = 0; ci < kCW; ++ci) {
            if (ci >= wr.chunks) continue;
            const uint32_t v = uint32_t(ci * wr.width + wr.lane);
            in[ci].w = row_ld_f32(r_master, v);
            if constexpr (kMomQ8) {
                if (!wide) {
                    in[ci].mc = row_ld_codes<kCodePolicy>(r_m, v);
                    in[ci].vc = row_ld_codes<kCodePolicy>(r_v, v);
                }
            } else {
                in[ci].mf = row_ld_f32(r_m, v);
                in[ci].vf = row_ld_f32(r_v, v);
            }
            if constexpr (kGrad == kQGradBf16) in[ci].gb = row_ld_bf16(r_g, v);
            if constexpr (kGrad == kQGradF32) in[ci].g4 = row_ld_f32(r_g, v);
            if constexpr (kGrad == kQGradQ8) in[ci].gc = row_ld_codes<kCodePolicy>(r_g, v);
            if (has_delta) in[ci].o2 = row_ld_bf16(r_o, v);
        }

        f32x4 mf[kCW], vf[kCW];
        uint32_t amax[2] = {0, 0};
#pragma unroll
        for (int ci = 0; ci < kCW; ++ci) {
            if (ci >= wr.chunks) continue;
            const uint32_t v = uint32_t(ci * wr.width + wr.lane);
            f32x4 w, d;
            step_math(in[ci], has_delta, ms, vs, gs, w, mf[ci], vf[ci], d);
            row_st_f32(r_master, v, w);
            row_st_bf16(r_w, v, w);
            if (has_delta) row_st_f32(r_d, v, d);
            if constexpr (!kMomQ8) {
                row_st_f32(r_m, v, mf[ci]);
                row_st_f32(r_v, v, vf[ci]);
            }
            if (kMomQ8 && int32_t(v) < wr.nvec) {
                amax[0] = absmax4(amax[0], mf[ci], 4);
                amax[1] = absmax4(amax[1], vf[ci], 4);
            }
        }
        if constexpr (!kMomQ8) return;

        // requantize the moments against the new row scales
        wave_team_max<kThreads, 2>(amax, wr.width);
        if (wr.len == 0) return;
        const QuantRow qm = quant_row(amax[0]), qv = quant_row(amax[1]);
        uint32_t cm[kCW], cv[kCW];
        quant_lane<kCW>(qm, mf, wr.chunks, cm);
        quant_lane<kCW>(qv, vf, wr.chunks, cv);
        if (wide) {
#pragma unroll
            for (int ci = 0; ci < kCW; ++ci) {
                if (ci >= wr.chunks) continue;
                stage[(ci >> 2) * 256 + (ci & 3) * 64 + j] = cm[ci];
                stage[(kStageGroups + (ci >> 2)) * 256 + (ci & 3) * 64 + j] = cv[ci];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                if (4 * g + (j >> 4) >= wr.chunks) continue;
                const u32x4_t qm4 = *reinterpret_cast<const u32x4_t *>(stage + g * 256 + 4 * j);
                const u32x4_t qv4 =
                    *reinterpret_cast<const u32x4_t *>(stage + (kStageGroups + g) * 256 + 4 * j);
                __builtin_amdgcn_raw_buffer_store_b128(qm4, r_m, wide_off(g), 0, kRowPolicy);
                __builtin_amdgcn_raw_buffer_store_b128(qv4, r_v, wide_off(g), 0, kRowPolicy);
            }
        } else {
#pragma unroll
            for (int ci = 0; ci < kCW; ++ci) {
                if (ci >= wr.chunks) continue;
                const uint32_t v = uint32_t(ci * wr.width + wr.lane);
                row_st_codes(r_m, v, cm[ci]);
                row_st_codes(r_v, v, cv[ci]);
            }
        }
        if (wr.lane == 0) {
            as_global<gfloat>(r.p[2])[wr.row] = qm.s;
            as_global<gfloat>(r.p[4])[wr.row] = qv.s;
        }
    }

    __device__ __forceinline__ void operator()(const Q8Rec &r, uint32_t local_block) const {
        if constexpr (kRows == kQRowsPacked) {   // kernels of their own: the paths differ
            packed_rows(r, local_block);         // in registers
            return;
        }
        if constexpr (kRows == kQRowsWave) {
            wave_rows<kC>(r, local_block);
            return;
        }
        if constexpr (kRows == kQRowsMixed) {
            // the record decides, for the whole workgroup (so a team's
            // barrier is reached by every lane or none); rows that fit the
            // separate launches' chunk count keep that loop's code
            if (r.flags & kQPacked)
                packed_rows(r, local_block);
            else if (r.chunks <= kC)
                wave_rows<kC>(r, local_block);
            else
                wave_rows<kQMixedWaveChunks>(r, local_block);
            return;
        }
        Row R{r.p[0], r.p[1], r.p[2], r.p[3], r.p[4], r.p[5], r.p[6], r.p[7], r.p[8], r.p[9],
              kDelta && r.p[9] != 0, 0.0f, 0.0f, 0.0f};
        const Team t = team_of<kThreads>(r, local_block);
        const bool has_row = t.len > 0;
        if (has_row) {
            if constexpr (kMomQ8) {
                R.ms = as_global<gfloat>(R.m_scale)[t.row];
                R.vs = as_global<gfloat>(R.v_scale)[t.row];
            }
            if constexpr (kGrad == kQGradQ8) R.gs = as_global<gfloat>(R.grad_scale)[t.row];
        }

        f32x4 mf[kC], vf[kC];
        uint32_t am = 0, av = 0;
        if (t.full)
            step_lane<true>(t, R, mf, vf, am, av);
        else
            step_lane<false>(t, R, mf, vf, am, av);
        if constexpr (!kMomQ8) return;

        // requantize the moments against the new row scales
        team_max2<kThreads>(t, am, av);
        if (!has_row) return;
        const QuantRow qm = quant_row(am), qv = quant_row(av);
        if (t.full) {
            quantize_store<kC, true>(t, R.m, qm, mf);
            quantize_store<kC, true>(t, R.v, qv, vf);
        } else {
            quantize_store<kC, false>(t, R.m, qm, mf);
            quantize_store<kC, false>(t, R.v, qv, vf);
        }
        if (t.lane == 0) {
            as_global<gfloat>(R.m_scale)[t.row] = qm.s;
            as_global<gfloat>(R.v_scale)[t.row] = qv.s;
        }
    }
};

// The mixed launch takes its record as a copy loaded up front, the others
// by reference (each field loaded where first used): on MI355X the copy
// brought the mixed kernel from 159 to 153 VGPRs and the rank-16 LoRA step
// about 2% faster, but the wave-row step over the Llama-2-7B attention
// projections 3% slower.
template <bool kMomQ8, QGrad kGrad, bool kDelta, int kThreads, int kRows>
__global__ __launch_bounds__(kThreads) void adamw_q8_kernel(const void *table, int nseg,
                                                            uint32_t block0, AdamwConsts c) {
    if constexpr (kRows == kQRowsMixed)
        block_of_table<Q8Rec>((ktable_t)table, nseg, block0,
                              AdamwRows<kMomQ8, kGrad, kDelta, kThreads, kRows>{c});
    else
        block_of_table<Q8Rec>(table, nseg, block0,
                              AdamwRows<kMomQ8, kGrad, kDelta, kThreads, kRows>{c});
}

// ------------------------------------------------------ accumulation

// int8 accumulator and one bf16 micro-batch: {codes, scale, grad_bf16}.
//   overwrite : acc = Q(f32(g))
//   otherwise : acc = Q(D(acc) + f32(g))
// The same team pattern serves the plain conversions of whole tensors:
// quantize {x, codes, scale} and dequantize (codes, scale -> x).
enum RowOp : int { kAccumAdd = 0, kAccumOverwrite = 1, kQuantize = 2, kDequantize = 3 };

template <RowOp kOp, int kThreads, int kRows>
struct CodeRows {
    static constexpr int kC = kRows == kQRowsWave     ? kQWaveCodeChunks
                              : kThreads == kQBlockWide ? kQWideChunks
                                                        : kQCodeChunks;
    static constexpr bool kAccum = kOp == kAccumAdd || kOp == kAccumOverwrite;
    static constexpr bool kReadsCodes = kOp == kAccumAdd || kOp == kDequantize;

    // The new accumulator values of one chunk: f32(g) on overwrite, else the
    // dequantized old value plus f32(g) (one binary32 addition each).
    __device__ __forceinline__ static f32x4 accumulated(uint32_t codes, u32x2 grad, float s_old) {
        const f32x4 g = widen_bf16(grad);
        if constexpr (kOp == kAccumOverwrite) return g;
        f32x4 x;
        for (int k = 0; k < 4; ++k) x[k] = accum_elem(dequant(code_at(codes, k), s_old), g[k], false);
        return x;
    }

    __device__ __forceinline__ static f32x4 dequantized(uint32_t codes, float s) {
        f32x4 d;
        for (int k = 0; k < 4; ++k) d[k] = dequant(code_at(codes, k), s);
        return d;
    }

    // The lane's new values (and their absmax), or for kDequantize the stores.
    template <bool kFull>
    __device__ __forceinline__ void values_lane(const Team &t, uint64_t codes, uint64_t src,
                                                float s_old, f32x4 (&x)[kC],
                                                uint32_t &amax) const {
        uint32_t cw[kC];
        u32x2 gb[kC];
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            x[ci] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const int64_t valid = valid_of<kFull>(t, ci);
            if (valid <= 0) continue;
            const int64_t e = t.first + chunk_off(t, ci);
            const bool vector = kFull || (t.vec && valid == 4);
            if constexpr (kReadsCodes) cw[ci] = load_codes(codes, e, vector, valid);
            if constexpr (kAccum) gb[ci] = load_bf16_bits(src, e, vector, valid);
            if constexpr (kOp == kQuantize) x[ci] = load_f32(src, e, vector, valid);
        }
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            const int64_t valid = valid_of<kFull>(t, ci);
            if (valid <= 0) continue;
            if constexpr (kAccum) x[ci] = accumulated(cw[ci], gb[ci], s_old);
            if constexpr (kOp == kDequantize) {
                const int64_t e = t.first + chunk_off(t, ci);
                store_f32(src, e, kFull || (t.vec && valid == 4), valid, dequantized(cw[ci], s_old));
            } else {
                amax = absmax4(amax, x[ci], valid);
            }
        }
    }

    // Packed rows: each chunk is a row of its own (see Packed).
    __device__ __forceinline__ void packed_rows(const Q8Rec &r, uint32_t local_block) const {
        const uint64_t codes = kAccum ? r.p[0] : r.p[1];
        const uint64_t scale = kAccum ? r.p[1] : r.p[2];
        const uint64_t src = kAccum ? r.p[2] : r.p[0];
        const Packed p = packed_of<kThreads, kC>(r, local_block);
        PackedChunk k[kC];
        float s_old[kC];
        uint32_t cw[kC];
        u32x2 gb[kC];
        f32x4 x[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            k[c] = packed_chunk(p, r, c);
            s_old[c] = 0.0f;
            if (kReadsCodes && k[c].has_row) s_old[c] = as_global<gfloat>(scale)[k[c].row];
            x[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const int64_t valid = k[c].valid;
            if (valid <= 0) continue;
            const bool vector = valid == 4;
            if constexpr (kReadsCodes) cw[c] = load_codes(codes, k[c].e, vector, valid);
            if constexpr (kAccum) gb[c] = load_bf16_bits(src, k[c].e, vector, valid);
            if constexpr (kOp == kQuantize) x[c] = load_f32(src, k[c].e, vector, valid);
        }
        uint32_t amax[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            amax[c] = 0;
            const int64_t valid = k[c].valid;
            if (valid <= 0) continue;
            if constexpr (kAccum) x[c] = accumulated(cw[c], gb[c], s_old[c]);
            if constexpr (kOp == kDequantize) {
                store_f32(src, k[c].e, valid == 4, valid, dequantized(cw[c], s_old[c]));
            } else {
                amax[c] = absmax4(0u, x[c], valid);
            }
        }
        if constexpr (kOp == kDequantize) return;
#pragma unroll
        for (int c = 0; c < kC; ++c) amax[c] = group_max(amax[c], p.width);
#pragma unroll
        for (int c = 0; c < kC; ++c) {
            if (!k[c].has_row) continue;
            const QuantRow q = quant_row(amax[c]);
            if (k[c].valid > 0)
                store_codes(codes, k[c].e, k[c].valid == 4, k[c].valid, quant_chunk(q, x[c]));
            if (p.lane == 0) as_global<gfloat>(scale)[k[c].row] = q.s;
        }
    }

    // Wave rows (see WaveRow).
    __device__ __forceinline__ void wave_rows(const Q8Rec &r, uint32_t local_block) const {
        const uint64_t codes = kAccum ? r.p[0] : r.p[1];
        const uint64_t scale = kAccum ? r.p[1] : r.p[2];
        const uint64_t src = kAccum ? r.p[2] : r.p[0];
        const WaveRow wr = wave_row_of<kThreads>(r, local_block);
        const auto rc = row_rsrc<1>(codes, wr);
        const auto rs = row_rsrc<kAccum ? 2 : 4>(src, wr);
        float s_old = 0.0f;
        if (kReadsCodes && wr.len > 0) s_old = as_global<gfloat>(scale)[wr.row];

        // chunks past wr.chunks are never read: no initialization for them
        uint32_t cw[kC];
        u32x2 gb[kC];
        f32x4 x[kC];
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            if (ci >= wr.chunks) continue;
            const uint32_t v = uint32_t(ci * wr.width + wr.lane);
            if constexpr (kReadsCodes) cw[ci] = row_ld_codes<kCodeLoadPolicy>(rc, v);
            if constexpr (kAccum) gb[ci] = row_ld_bf16(rs, v);
            if constexpr (kOp == kQuantize) x[ci] = row_ld_f32(rs, v);
        }
        uint32_t amax[1] = {0};
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            if (ci >= wr.chunks) continue;
            const uint32_t v = uint32_t(ci * wr.width + wr.lane);
            if constexpr (kAccum) x[ci] = accumulated(cw[ci], gb[ci], s_old);
            if constexpr (kOp == kDequantize) {
                row_st_f32(rs, v, dequantized(cw[ci], s_old));
            } else if (int32_t(v) < wr.nvec) {
                amax[0] = absmax4(amax[0], x[ci], 4);
            }
        }
        if constexpr (kOp == kDequantize) return;

        wave_team_max<kThreads, 1>(amax, wr.width);
        if (wr.len == 0) return;
        const QuantRow q = quant_row(amax[0]);
        uint32_t w[kC];
        quant_lane<kC>(q, x, wr.chunks, w);
#pragma unroll
        for (int ci = 0; ci < kC; ++ci) {
            if (ci >= wr.chunks) continue;
            row_st_codes(rc, uint32_t(ci * wr.width + wr.lane), w[ci]);
        }
        if (wr.lane == 0) as_global<gfloat>(scale)[wr.row] = q.s;
    }

    __device__ __forceinline__ void operator()(const Q8Rec &r, uint32_t local_block) const {
        if constexpr (kRows == kQRowsPacked) {   // kernels of their own: the paths differ
            packed_rows(r, local_block);         // in registers
            return;
        }
        if constexpr (kRows == kQRowsWave) {
            wave_rows(r, local_block);
            return;
        }
        const Team t = team_of<kThreads>(r, local_block);
        const bool has_row = t.len > 0;
        // pointers: accumulation {codes, scale, grad}; conversions {x, codes, scale}
        const uint64_t codes = kAccum ? r.p[0] : r.p[1];
        const uint64_t scale = kAccum ? r.p[1] : r.p[2];
        const uint64_t src = kAccum ? r.p[2] : r.p[0];

        float s_old = 0.0f;
        if (has_row && kReadsCodes) s_old = as_global<gfloat>(scale)[t.row];

        f32x4 x[kC];
        uint32_t amax = 0, unused = 0;
        if (t.full)
            values_lane<true>(t, codes, src, s_old, x, amax);
        else
            values_lane<false>(t, codes, src, s_old, x, amax);
        if constexpr (kOp == kDequantize) return;

        team_max2<kThreads>(t, amax, unused);
        if (!has_row) return;
        const QuantRow q = quant_row(amax);
        if (t.full)
            quantize_store<kC, true>(t, codes, q, x);
        else
            quantize_store<kC, false>(t, codes, q, x);
        if (t.lane == 0) as_global<gfloat>(scale)[t.row] = q.s;
    }
};

template <RowOp kOp, int kThreads, int kRows>
__global__ __launch_bounds__(kThreads) void code_rows_kernel(const void *table, int nseg,
                                                             uint32_t block0) {
    block_of_table<Q8Rec>(table, nseg, block0, CodeRows<kOp, kThreads, kRows>{});
}

// row_reciprocal over n scales (a measurement aid: its error bound is what
// the division-free quantization relies on).  Grid-stride over n.
__global__ __launch_bounds__(256) void q8_recip_probe_kernel(const float *__restrict__ s,
                                                             float *__restrict__ r, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * 256)
        r[i] = row_reciprocal(s[i]);
}

// `lds` bytes of dynamic LDS are reserved per workgroup (none of these
// kernels reads them): a cap on how many workgroups share a CU.
template <class... Args>
hipError_t launch_split(const void *fn, int block, uint32_t total_blocks, uint32_t lds,
                        hipStream_t stream, const void *table, int nseg, Args... extra) {
    for (uint32_t block0 = 0; block0 < total_blocks;) {
        const uint32_t n = std::min<uint32_t>(total_blocks - block0, max_blocks_per_launch(block));
        void *args[] = {&table, &nseg, &block0, &extra...};
        hipError_t e = hipLaunchKernel(fn, dim3(n), dim3(block), args, lds, stream);
        if (e != hipSuccess) return e;
        block0 += n;
    }
    return hipSuccess;
}

// Kernels per launch group: row teams, wave rows (kQBlock- or kQBlockWide-
// lane workgroups) or packed rows (kQBlock lanes only).
template <bool kMomQ8, QGrad kGrad, bool kDelta, int kRows>
const void *pick_adamw_rows(int block) {
    return block == kQBlock
               ? reinterpret_cast<const void *>(&adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlock, kRows>)
               : reinterpret_cast<const void *>(
                     &adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlockWide, kRows>);
}

template <bool kMomQ8, QGrad kGrad, bool kDelta>
const void *pick_adamw(int block, QRows rows) {
    switch (rows) {
    case kQRowsPacked:
        return reinterpret_cast<const void *>(
            &adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlock, kQRowsPacked>);
    case kQRowsMixed:
        return reinterpret_cast<const void *>(
            &adamw_q8_kernel<kMomQ8, kGrad, kDelta, kQBlock, kQRowsMixed>);
    case kQRowsWave: return pick_adamw_rows<kMomQ8, kGrad, kDelta, kQRowsWave>(block);
    default: return pick_adamw_rows<kMomQ8, kGrad, kDelta, kQRowsTeam>(block);
    }
}

template <bool kMomQ8, QGrad kGrad>
const void *pick_adamw_delta(bool with_delta, int block, QRows rows) {
    return with_delta ? pick_adamw<kMomQ8, kGrad, true>(block, rows)
                      : pick_adamw<kMomQ8, kGrad, false>(block, rows);
}

// Accumulation and conversions: wave rows and packed rows run in kQBlock-lane
// workgroups only (wave rows hold up to kQWaveCodeChunks chunks per lane).
template <RowOp kOp>
const void *pick_rows(int block, QRows rows) {
    switch (rows) {
    case kQRowsPacked:
        return reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlock, kQRowsPacked>);
    case kQRowsWave:
        return reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlock, kQRowsWave>);
    default:
        return block == kQBlock
                   ? reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlock, kQRowsTeam>)
                   : reinterpret_cast<const void *>(&code_rows_kernel<kOp, kQBlockWide, kQRowsTeam>);
    }
}

// Families of the step kernels and the workgroup sizes they come in.
bool block_ok(int block, QRows rows) {
    if (rows == kQRowsMixed) return block == kQBlock;
    if (rows != kQRowsTeam && rows != kQRowsPacked && rows != kQRowsWave) return false;
    return block == kQBlock || (block == kQBlockWide && rows != kQRowsPacked);
}

// ... and of the accumulation and conversion kernels (no mixed launches).
bool rows_block_ok(int block, QRows rows) {
    return rows != kQRowsMixed && block_ok(block, rows) && (block == kQBlock || rows == kQRowsTeam);
}

}  // namespace

const void *adamw_q8_kernel_fn(bool moments_q8, QGrad grad, bool with_delta, int block,
                               QRows rows) {
    if (!block_ok(block, rows)) return nullptr;
    if (moments_q8) {
        switch (grad) {
        case kQGradBf16: return pick_adamw_delta<true, kQGradBf16>(with_delta, block, rows);
        case kQGradF32: return pick_adamw_delta<true, kQGradF32>(with_delta, block, rows);
        case kQGradQ8: return pick_adamw_delta<true, kQGradQ8>(with_delta, block, rows);
        default: return nullptr;
        }
    }
    // fp32 moments only pair with an int8 gradient here; the other
    // combinations run on the tile kernels of lema_kernels.hip
    if (grad != kQGradQ8) return nullptr;
    return pick_adamw_delta<false, kQGradQ8>(with_delta, block, rows);
}

hipError_t launch_adamw_q8(const void *table, int nseg, uint32_t total_blocks, bool moments_q8,
                           QGrad grad, bool with_delta, int block, QRows rows,
                           const AdamwConsts &c, hipStream_t stream, uint32_t lds_bytes) {
    const void *fn = adamw_q8_kernel_fn(moments_q8, grad, with_delta, block, rows);
    if (fn == nullptr) return hipErrorInvalidValue;
    return launch_split(fn, block, total_blocks, lds_bytes, stream, table, nseg, c);
}

hipError_t launch_accum_q8(const void *table, int nseg, uint32_t total_blocks, bool overwrite,
                           int block, QRows rows, hipStream_t stream) {
    if (!rows_block_ok(block, rows)) return hipErrorInvalidValue;
    const void *fn = overwrite ? pick_rows<kAccumOverwrite>(block, rows)
                               : pick_rows<kAccumAdd>(block, rows);
    return launch_split(fn, block, total_blocks, 0, stream, table, nseg);
}

hipError_t launch_quantize_q8(const void *table, int nseg, uint32_t total_blocks, bool dequantize,
                              int block, QRows rows, hipStream_t stream) {
    if (!rows_block_ok(block, rows)) return hipErrorInvalidValue;
    const void *fn = dequantize ? pick_rows<kDequantize>(block, rows)
                                : pick_rows<kQuantize>(block, rows);
    return launch_split(fn, block, total_blocks, 0, stream, table, nseg);
}

hipError_t launch_q8_recip_probe(const float *s, float *r, int64_t n, hipStream_t stream) {
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536));
    void *args[] = {&s, &r, &n};
    return hipLaunchKernel(reinterpret_cast<const void *>(&q8_recip_probe_kernel),
                           dim3(unsigned(blocks)), dim3(256), args, 0, stream);
}

}  // namespace lema
