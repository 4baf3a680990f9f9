// lema_noalloc.hip -- lema_adamw_step_noalloc: the AdamW step of
// lema_adamw_step for callers that cannot allocate device memory.
//
// lema_adamw_step keeps its launch tables in a per-device cache whose
// entries it allocates on first use.  This entry point instead writes the
// table into `scratch`, a fixed array of device memory in this file's code
// object: each GPU the library runs on holds its own copy from the moment
// the code object is loaded until the process ends.  The table reaches the
// array through the kernel arguments of a small copy kernel (2 KiB per
// launch, stream-ordered), so no host buffer has to outlive the call and no
// memory is allocated on the host or on the device.  The step itself is the
// same adamw_tile_kernel launch, with the same occupancy reservation, as
// lema_adamw_step's.
//
// Every call on one GPU shares that GPU's array and leaves its table there;
// calls on the same stream are ordered, calls that overlap on one GPU on
// different streams race for it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "lema.h"
#include "lema_host_internal.h"
#include "lema_internal.h"

namespace lema {
namespace {

constexpr int kNoAllocMaxSegs = LEMA_NOALLOC_MAX_SEGMENTS;
constexpr size_t kScratchBytes = (table_bytes(kNoAllocMaxSegs) + 255) & ~size_t(255);
static_assert(kScratchBytes <= 128 * 1024, "the no-allocation table stays modest");

}  // namespace
}  // namespace lema

// The launch table of lema_adamw_step_noalloc: one copy per GPU.  Host code
// uses the address hipGetSymbolAddress returns for the current device, never
// this name.
static __device__ __align__(256) unsigned char scratch[lema::kScratchBytes];

namespace lema {
namespace {

// One piece of a launch table, carried by value in the kernel arguments.
constexpr uint32_t kChunkBytes = 2048;
struct TableChunk {
    uint4 w[kChunkBytes / 16];
};

// dst[0 .. nbytes) = chunk (nbytes a multiple of 16, at most kChunkBytes).
__global__ __launch_bounds__(64) void table_chunk_kernel(uint4 *__restrict__ dst, uint32_t nwords,
                                                         TableChunk chunk) {
    for (uint32_t i = threadIdx.x; i < nwords; i += 64) dst[i] = chunk.w[i];
}

constexpr int kMaxDevices = 64;

std::mutex g_mu;                      // guards everything below
void *g_scratch[kMaxDevices];         // per device: the address of `scratch`
bool g_scratch_ready[kMaxDevices];
// host image of the table being written, and the spans of its validation
alignas(64) unsigned char g_image[kScratchBytes];
Span g_spans[size_t(kNoAllocMaxSegs) * 7];

// The device address of `scratch` on the current device (looked up on the
// first call there, with that device current).
lema_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    if (dev < 0 || dev >= kMaxDevices) return LEMA_ERR_SIZE;
    if (!g_scratch_ready[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_failed(e);
        if (p == nullptr) return hip_failed(hipErrorInvalidSymbol);
        g_scratch[dev] = p;
        g_scratch_ready[dev] = true;
    }
    *out = g_scratch[dev];
    return LEMA_OK;
}

// Lays the non-empty segments out as a launch table in g_image; returns its
// bytes, and the tile count and whether any segment writes a delta.
size_t build_image(const lema_adamw_seg *segs, int32_t nseg, uint64_t *tiles, bool *with_delta,
                   int *nrec) {
    int n = 0;
    for (int32_t i = 0; i < nseg; ++i) n += segs[i].numel > 0;
    const size_t bytes = table_bytes(n);
    std::memset(g_image, 0, bytes);
    uint32_t *tile_begin = reinterpret_cast<uint32_t *>(g_image);
    SegRec *recs = reinterpret_cast<SegRec *>(g_image + table_tiles_bytes(n));
    uint64_t t = 0;
    int k = 0;
    *with_delta = false;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_seg &s = segs[i];
        if (s.numel == 0) continue;
        SegRec &r = recs[k];
        r.p[0] = reinterpret_cast<uint64_t>(s.master);
        r.p[1] = reinterpret_cast<uint64_t>(s.exp_avg);
        r.p[2] = reinterpret_cast<uint64_t>(s.exp_avg_sq);
        r.p[3] = reinterpret_cast<uint64_t>(s.grad);
        r.p[4] = reinterpret_cast<uint64_t>(s.weight_bf16);
        r.p[5] = reinterpret_cast<uint64_t>(s.orig_bf16);
        r.p[6] = reinterpret_cast<uint64_t>(s.delta);
        r.numel = s.numel;
        *with_delta |= s.delta != nullptr;
        tile_begin[k] = static_cast<uint32_t>(t);
        t += static_cast<uint64_t>((s.numel + kTile - 1) / kTile);
        ++k;
    }
    tile_begin[n] = static_cast<uint32_t>(t);
    *tiles = t;
    *nrec = n;
    return bytes;
}

}  // namespace
}  // namespace lema

using namespace lema;

extern "C" lema_status lema_adamw_step_noalloc(const lema_adamw_seg *segs, int32_t nseg,
                                               const lema_adamw_args *args, void *stream_) {
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (nseg < 0 || nseg > kNoAllocMaxSegs) return LEMA_ERR_SIZE;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    std::lock_guard<std::mutex> lock(g_mu);
    FixedSpans spans{g_spans, sizeof(g_spans) / sizeof(g_spans[0])};
    st = validate_adamw_segs(segs, nseg, args->grad_dtype, true, &spans);
    if (st != LEMA_OK) return st;
    if (spans.overflow) return LEMA_ERR_SIZE;
    if (any_conflict(spans.data, spans.data + spans.n)) return LEMA_ERR_OVERLAP;
    uint64_t tiles = 0;
    bool with_delta = false;
    int nrec = 0;
    const size_t bytes = build_image(segs, nseg, &tiles, &with_delta, &nrec);
    if (tiles > kMaxTiles) return LEMA_ERR_SIZE;
    if (nrec == 0) return LEMA_OK;

    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &capture);
    if (e != hipSuccess) return hip_failed(e);
    if (capture != hipStreamCaptureStatusNone) return LEMA_ERR_CAPTURE;
    void *table = nullptr;
    st = scratch_address(&table);
    if (st != LEMA_OK) return st;
    // bytes <= kScratchBytes: nseg is at most kNoAllocMaxSegs
    for (size_t off = 0; off < bytes; off += kChunkBytes) {
        const uint32_t n = static_cast<uint32_t>(std::min<size_t>(kChunkBytes, bytes - off));
        TableChunk chunk;
        std::memcpy(chunk.w, g_image + off, n);
        uint4 *dst = reinterpret_cast<uint4 *>(static_cast<unsigned char *>(table) + off);
        uint32_t nwords = n / 16;
        void *kargs[] = {&dst, &nwords, &chunk};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&table_chunk_kernel), dim3(1), dim3(64),
                            kargs, 0, stream);
        if (e != hipSuccess) return hip_failed(e);
    }
    const GradMode mode = args->grad_dtype == LEMA_GRAD_FP32 ? kGradF32 : kGradBf16;
    e = launch_adamw(table, nullptr, nrec, static_cast<uint32_t>(tiles), mode, with_delta,
                     derive_consts(args), stream, 0, step_lds_bytes_for(mode, with_delta, 0, tiles));
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}
