// lema_device.h -- device helpers shared by the gfx950 kernel files: vector
// types, global-address-space access, bf16 conversion, the per-element AdamW
// arithmetic and the tile -> segment lookup of the launch tables.
#pragma once

#include <hip/hip_runtime.h>

#include "lema_internal.h"

namespace lema {
namespace dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Pointers into global memory (address space 1).  The segment pointers come
// out of LDS, so without this the compiler could not prove where they point
// and would emit flat instructions instead of global loads and stores.
#define LEMA_GLOBAL __attribute__((address_space(1)))
typedef LEMA_GLOBAL float gfloat;
typedef LEMA_GLOBAL uint16_t gu16;
typedef LEMA_GLOBAL f32x4 gf32x4;
typedef LEMA_GLOBAL u32x2 gu32x2;

template <class T>
__device__ __forceinline__ T *as_global(uint64_t addr) {
    return reinterpret_cast<T *>(addr);
}

// ------------------------------------------------------------- helpers

// bf16 is the upper half of an fp32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_one(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two fp32 -> a pair of bf16, nearest-even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t to_bf16_pair(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 b = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint16_t to_bf16_one(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// One AdamW element (the arithmetic stated in include/lema.h).
__device__ __forceinline__ void adamw_elem(float &w, float &m, float &v, float g,
                                           const AdamwConsts &c) {
#pragma clang fp contract(off)
    const float w_decayed = w * c.decay;
    const float m_new = c.b1 * m + c.omb1 * g;
    const float v_new = c.b2 * v + c.omb2 * (g * g);
    const float denom = __builtin_sqrtf(v_new) * c.inv_bc2_root + c.eps;
    w = w_decayed - c.step_size * (m_new / denom);
    m = m_new;
    v = v_new;
}

__device__ __forceinline__ float accum_elem(float acc, float g, bool overwrite) {
#pragma clang fp contract(off)
    return overwrite ? g : acc + g;
}

// ---------------------------------------------------------- segment lookup

// Nontemporal vector loads and stores through global-address-space pointers.
template <class T>
__device__ __forceinline__ T ld_nt(uint64_t base, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const LEMA_GLOBAL T *>(base) + i);
}
template <class T>
__device__ __forceinline__ void st_nt(uint64_t base, int64_t i, T v) {
    __builtin_nontemporal_store(v, reinterpret_cast<LEMA_GLOBAL T *>(base) + i);
}

// Tile-scoped vector accesses of the tile kernels, through a buffer resource
// whose base is the tile's first vector in one array and whose size is the
// tile's bytes: the 64-bit base stays in scalar registers, each lane adds a
// small 32-bit offset, and the hardware range check keeps every access
// inside the tile.  Cache policy (gfx950 bits SC0 = 1, NT = 2, SC1 = 16):
// nontemporal loads and nontemporal SC1 stores.  Measured on one MI355X for
// the AdamW step over Llama-2-7B q,k,v,o: 1.526-1.623 ms, against
// 1.593-1.664 ms for nontemporal global instructions in the same runs.  NT
// stores reached 1.546-1.650, SC1 alone 1.621-1.630, plain loads 1.675.
// Accumulation gained 10% and merge_delta 8%.
constexpr int kTileLoadPolicy = 2;
constexpr int kTileStorePolicy = 2 | 16;
constexpr int kRawBufferWord3 = 0x00020000;   // raw (untyped) buffer on gfx9

template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(uint64_t array, int64_t first_vec,
                                                           int nvec) {
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(array + uint64_t(first_vec) * sizeof(T)), 0,
        int(nvec * sizeof(T)), kRawBufferWord3);
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Vector `lane` of a tile (T is 16 or 8 bytes).
template <class T>
__device__ __forceinline__ T tile_ld(__amdgpu_buffer_rsrc_t r, int lane) {
    const int off = lane * int(sizeof(T));
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kTileLoadPolicy));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kTileLoadPolicy));
}

template <class T>
__device__ __forceinline__ void tile_st(__amdgpu_buffer_rsrc_t r, int lane, T v) {
    const int off = lane * int(sizeof(T));
    if constexpr (sizeof(T) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0,
                                               kTileStorePolicy);
    else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, off, 0,
                                              kTileStorePolicy);
}

// Launch tables are read through the constant address space, whether they
// sit in device memory or in the kernel arguments: their reads are uniform
// over a wavefront and stay scalar loads.
#define LEMA_CONST __attribute__((address_space(4)))
typedef const LEMA_CONST unsigned char *ktable_t;

// The launch table of a tile kernel: the device copy when `table` is set,
// else the copy carried in the kernel arguments (a by-value kernel argument
// lives in the kernel-argument segment, so `inl` is read in place there).
__device__ __forceinline__ ktable_t launch_table(const void *table, const InlineTable &inl) {
    return table != nullptr ? (ktable_t)table : (ktable_t)&inl;
}

// A record read from a launch table, one 8-byte word at a time.
template <class Rec>
__device__ __forceinline__ Rec table_record(ktable_t recs, int s) {
    static_assert(sizeof(Rec) % 8 == 0, "records are whole 8-byte words");
    struct Words {
        uint64_t w[sizeof(Rec) / 8];
    } out;
    const LEMA_CONST uint64_t *src = (const LEMA_CONST uint64_t *)(recs + sizeof(Rec) * size_t(s));
#pragma unroll
    for (size_t i = 0; i < sizeof(Rec) / 8; ++i) out.w[i] = src[i];
    return __builtin_bit_cast(Rec, out);
}

// The segment holding tile t: the last s with tile_begin[s] <= t.  The
// table guarantees tile_begin[0] = 0 <= t < tile_begin[nseg].
template <class Begin>
__device__ __forceinline__ int find_segment(Begin tile_begin, int nseg, uint32_t t) {
    int lo = 0, hi = nseg;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_begin[mid] <= t)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Run fn(record, block-within-segment) for the block of this workgroup.
// Table layout: uint32_t begin[nseg + 1] (prefix sums of blocks per segment),
// padded to 64 bytes, then Rec[nseg].
template <class Rec, class Fn>
__device__ __forceinline__ void block_of_table(ktable_t table, int nseg, uint32_t block0,
                                               const Fn &fn) {
    const LEMA_CONST uint32_t *begin = (const LEMA_CONST uint32_t *)table;
    const uint32_t t = block0 + blockIdx.x;
    const int s = find_segment(begin, nseg, t);
    fn(table_record<Rec>(table + table_tiles_bytes(nseg), s), t - begin[s]);
}

// The same for a table only ever in device memory (the int8 kernels): the
// record is passed by reference, so the compiler loads each field where the
// kernel first needs it.  The variant above copies the record, since its
// functors take generic references; copying the int8 kernels' 120-byte
// record up front that way measured 3% slower on the int8 step over the
// Llama-2-7B attention projections (MI355X, three interleaved rounds).
template <class Rec, class Fn>
__device__ __forceinline__ void block_of_table(const void *table, int nseg, uint32_t block0,
                                               const Fn &fn) {
    const uint32_t *begin = static_cast<const uint32_t *>(table);
    const Rec *recs = reinterpret_cast<const Rec *>(static_cast<const char *>(table) +
                                                    table_tiles_bytes(nseg));
    const uint32_t t = block0 + blockIdx.x;
    const int s = find_segment(begin, nseg, t);
    fn(recs[s], t - begin[s]);
}

}  // namespace dev
}  // namespace lema
