// lema_host.cpp -- host side of the C ABI in include/lema.h: argument
// validation, fp32 constant derivation, launch tables and kernel launches.
//
// Method: LEMA README, "Quick Start" (torch.optim.AdamW, lr 1e-4) and
// "Selective Full Fine-Tuning" (per-layer AdamW over fp32 states, fp32
// gradient accumulation, fp32 delta checkpoint); LLMScale fine-tuning VRAM
// page (16 bytes per trained parameter).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <vector>

#include "lema.h"
#include "lema_host_internal.h"
#include "lema_measure.h"
#include "lema_internal.h"

namespace lema {

static_assert(kMaxMicrobatches == LEMA_MAX_MICROBATCHES, "micro-batch limit of header and kernel");

// ------------------------------------------------------------ errors

static thread_local int32_t t_last_hip_error = 0;

lema_status hip_failed(hipError_t e) {
    t_last_hip_error = static_cast<int32_t>(e);
    return LEMA_ERR_HIP;
}

// ------------------------------------------------------- constants

// beta^t in double by square-and-multiply, taking the bits of t from the
// least significant end.
static double beta_pow(double beta, int64_t t) {
    double acc = 1.0;
    double sq = beta;
    for (int64_t e = t; e != 0; e >>= 1) {
        if (e & 1) acc *= sq;
        sq *= sq;
    }
    return acc;
}

lema_status check_hparams(const lema_adamw_args *a, bool allow_q8_grad) {
    if (a == nullptr) return LEMA_ERR_NULL;
    const double vals[] = {a->lr, a->beta1, a->beta2, a->eps, a->weight_decay};
    for (double x : vals)
        if (!std::isfinite(x)) return LEMA_ERR_HPARAM;
    if (a->lr < 0.0 || a->weight_decay < 0.0 || a->eps <= 0.0) return LEMA_ERR_HPARAM;
    if (a->beta1 < 0.0 || a->beta1 >= 1.0 || a->beta2 < 0.0 || a->beta2 >= 1.0) return LEMA_ERR_HPARAM;
    if (a->step < 1) return LEMA_ERR_HPARAM;
    if (a->reserved != 0) return LEMA_ERR_HPARAM;
    if (a->grad_dtype == LEMA_GRAD_BF16 || a->grad_dtype == LEMA_GRAD_FP32) return LEMA_OK;
    if (allow_q8_grad && a->grad_dtype == LEMA_GRAD_Q8) return LEMA_OK;
    return LEMA_ERR_DTYPE;
}

AdamwConsts derive_consts(const lema_adamw_args *a) {
    // each constant: computed in double, rounded to fp32 once
    const double bias1 = 1.0 - beta_pow(a->beta1, a->step);
    const double bias2 = 1.0 - beta_pow(a->beta2, a->step);
    AdamwConsts c;
    c.b1 = static_cast<float>(a->beta1);
    c.omb1 = static_cast<float>(1.0 - a->beta1);
    c.b2 = static_cast<float>(a->beta2);
    c.omb2 = static_cast<float>(1.0 - a->beta2);
    c.eps = static_cast<float>(a->eps);
    c.decay = static_cast<float>(1.0 - a->lr * a->weight_decay);
    c.step_size = static_cast<float>(a->lr / bias1);
    c.inv_bc2_root = static_cast<float>(1.0 / std::sqrt(bias2));
    return c;
}

// ------------------------------------------------------- validation

// True if two spans intersect and at least one of them is written.
bool any_conflict(Span *begin, Span *end) {
    std::sort(begin, end, [](const Span &x, const Span &y) { return x.lo < y.lo; });
    uintptr_t reach_any = 0, reach_written = 0;   // max end of spans seen so far
    bool seen = false;
    for (const Span *p = begin; p != end; ++p) {
        const Span &s = *p;
        if (seen) {
            if (reach_written > s.lo) return true;
            if (s.written && reach_any > s.lo) return true;
        }
        seen = true;
        reach_any = std::max(reach_any, s.hi);
        if (s.written) reach_written = std::max(reach_written, s.hi);
    }
    return false;
}

// A training loop hands the same arrays to every step, and sorting a few
// thousand spans costs more host time than a small step's kernel (448 LoRA
// tensors: about 4,500 spans, 180 us to sort on a 2.7 GHz Xeon).  So each
// thread keeps the last span list found free of conflicts, in the order it
// was given; an identical list, compared field by field, has the same
// answer without the sort.  A list with a conflict is never kept.
static bool same_spans(const std::vector<Span> &a, const std::vector<Span> &b) {
    if (a.size() != b.size()) return false;
    for (size_t i = 0; i < a.size(); ++i)
        if (a[i].lo != b[i].lo || a[i].hi != b[i].hi || a[i].written != b[i].written)
            return false;
    return true;
}

bool any_conflict(std::vector<Span> &spans) {
    constexpr size_t kRememberFrom = 64;   // below this the sort is cheaper than the copy
    if (spans.size() < kRememberFrom) return any_conflict(spans.data(), spans.data() + spans.size());
    thread_local std::vector<Span> last_clear;
    if (same_spans(spans, last_clear)) return false;
    std::vector<Span> given(spans);
    if (any_conflict(spans.data(), spans.data() + spans.size())) return true;
    last_clear.swap(given);
    return false;
}

template <class Spans>
static void push_span(Spans &spans, const void *p, int64_t numel, size_t elem, bool written) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    spans.push_back(Span{lo, lo + static_cast<uintptr_t>(numel) * elem, written});
}

void add_span(std::vector<Span> &spans, const void *p, int64_t numel, size_t elem,
              bool written) {
    push_span(spans, p, numel, elem, written);
}

template <class Spans>
static lema_status validate_adamw_segs_into(const lema_adamw_seg *segs, int32_t nseg,
                                            int32_t grad_dtype, bool delta_allowed,
                                            Spans *spans) {
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    const size_t gsize = grad_dtype == LEMA_GRAD_FP32 ? 4 : 2;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_seg &s = segs[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if ((s.orig_bf16 == nullptr) != (s.delta == nullptr)) return LEMA_ERR_NULL;
        if (!delta_allowed && s.delta != nullptr) return LEMA_ERR_NULL;
        if (s.numel == 0) continue;
        if (!s.master || !s.exp_avg || !s.exp_avg_sq || !s.grad || !s.weight_bf16) return LEMA_ERR_NULL;
        const uintptr_t f32 = reinterpret_cast<uintptr_t>(s.master) |
                              reinterpret_cast<uintptr_t>(s.exp_avg) |
                              reinterpret_cast<uintptr_t>(s.exp_avg_sq) |
                              reinterpret_cast<uintptr_t>(s.delta) |
                              (gsize == 4 ? reinterpret_cast<uintptr_t>(s.grad) : 0);
        const uintptr_t b16 = reinterpret_cast<uintptr_t>(s.weight_bf16) |
                              reinterpret_cast<uintptr_t>(s.orig_bf16) |
                              (gsize == 2 ? reinterpret_cast<uintptr_t>(s.grad) : 0);
        if ((f32 & 3) || (b16 & 1)) return LEMA_ERR_ALIGN;
        if (spans) {
            push_span(*spans, s.master, s.numel, 4, true);
            push_span(*spans, s.exp_avg, s.numel, 4, true);
            push_span(*spans, s.exp_avg_sq, s.numel, 4, true);
            push_span(*spans, s.grad, s.numel, gsize, false);
            push_span(*spans, s.weight_bf16, s.numel, 2, true);
            if (s.delta) {
                push_span(*spans, s.orig_bf16, s.numel, 2, false);
                push_span(*spans, s.delta, s.numel, 4, true);
            }
        }
    }
    return LEMA_OK;
}

lema_status validate_adamw_segs(const lema_adamw_seg *segs, int32_t nseg, int32_t grad_dtype,
                                bool delta_allowed, std::vector<Span> *spans) {
    return validate_adamw_segs_into(segs, nseg, grad_dtype, delta_allowed, spans);
}

lema_status validate_adamw_segs(const lema_adamw_seg *segs, int32_t nseg, int32_t grad_dtype,
                                bool delta_allowed, FixedSpans *spans) {
    return validate_adamw_segs_into(segs, nseg, grad_dtype, delta_allowed, spans);
}

// ----------------------------------------------- per-device state

namespace {

constexpr int kMaxDevices = 64;
// Tables kept per device.  A training loop that calls the library for every
// layer and micro-batch cycles through a few hundred distinct tables, and a
// cache smaller than that cycle misses on every call; entries cost 32 KiB
// (device table plus page-locked staging), so all of them are kept.
constexpr size_t kMaxCacheEntries = 512;

// A launch table kept on the device.  Tables are immutable once uploaded;
// a call whose table is byte-identical to a cached one launches on it
// without any copy (the usual case: the same tensors every step).
struct TableEntry {
    std::vector<unsigned char> bytes;
    uint64_t hash = 0;
    void *dev = nullptr;
    size_t dev_cap = 0;
    void *staging = nullptr;      // page-locked source of the upload
    size_t staging_cap = 0;
    hipEvent_t last_use = nullptr;
    hipStream_t last_stream = nullptr;
    bool recorded = false;        // last_use marks the entry's latest launch
    uint64_t stamp = 0;
};

struct DeviceState {
    std::mutex mu;
    bool ready = false;
    int cu_count = 0;
    int lds_per_cu = 0;           // bytes of LDS per compute unit
    uint64_t clock = 0;
    std::vector<std::unique_ptr<TableEntry>> entries;
    int64_t hits = 0, uploads = 0, waits = 0;
};

DeviceState g_devices[kMaxDevices];

// FNV-1a over the table's 8-byte words (then any tail bytes): a cheap first
// test before comparing bytes.
uint64_t table_hash(const std::vector<unsigned char> &bytes) {
    uint64_t h = 1469598103934665603ull;
    const size_t words = bytes.size() / 8;
    for (size_t i = 0; i < words; ++i) {
        uint64_t w;
        std::memcpy(&w, bytes.data() + 8 * i, 8);
        h = (h ^ w) * 1099511628211ull;
    }
    for (size_t i = 8 * words; i < bytes.size(); ++i) h = (h ^ bytes[i]) * 1099511628211ull;
    return h;
}

lema_status device_state(DeviceState **out, int *device) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    if (dev < 0 || dev >= kMaxDevices) return LEMA_ERR_SIZE;
    DeviceState &d = g_devices[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (!d.ready) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_failed(e);
        d.cu_count = cus > 0 ? cus : 1;
        int lds = 0;
        e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (e != hipSuccess) return hip_failed(e);
        d.lds_per_cu = lds;
        d.ready = true;
    }
    *out = &d;
    if (device) *device = dev;
    return LEMA_OK;
}

// True when no launch on the entry's table is still pending.
bool entry_idle(const TableEntry &t) {
    return !t.recorded || hipEventQuery(t.last_use) == hipSuccess;
}

// Pick the cache entry for `bytes` (must hold d.mu).  On a hit nothing is
// copied.  On a miss a new entry is added while there are fewer than
// kMaxCacheEntries; beyond that the least recently used entry whose launches
// have finished is reloaded, and only if all are pending does the call wait
// for the least recently used one.
lema_status acquire_table(DeviceState &d, const std::vector<unsigned char> &bytes,
                          hipStream_t stream, TableEntry **out) {
    hipError_t e;
    const uint64_t h = table_hash(bytes);
    for (auto &p : d.entries) {
        TableEntry &t = *p;
        if (!t.bytes.empty() && t.hash == h && t.bytes == bytes) {
            if (t.recorded && t.last_stream != stream) {
                // a later reload must wait for both streams' launches
                e = hipStreamWaitEvent(stream, t.last_use, 0);
                if (e != hipSuccess) return hip_failed(e);
            }
            *out = &t;
            ++d.hits;
            return LEMA_OK;
        }
    }
    ++d.uploads;
    TableEntry *victim = nullptr;
    if (d.entries.size() < kMaxCacheEntries) {
        d.entries.push_back(std::make_unique<TableEntry>());
        victim = d.entries.back().get();
    }
    if (!victim) {
        for (auto &p : d.entries)
            if (entry_idle(*p) && (!victim || p->stamp < victim->stamp)) victim = p.get();
    }
    if (!victim) {
        for (auto &p : d.entries)
            if (!victim || p->stamp < victim->stamp) victim = p.get();
        ++d.waits;
        e = hipEventSynchronize(victim->last_use);
        if (e != hipSuccess) return hip_failed(e);
    }
    victim->bytes.clear();
    const size_t n = bytes.size();
    if (victim->dev_cap < n) {
        if (victim->dev) (void)hipFree(victim->dev);
        victim->dev = nullptr;
        victim->dev_cap = 0;
        const size_t cap = std::max<size_t>(n, 16384);
        e = hipMalloc(&victim->dev, cap);
        if (e != hipSuccess) return hip_failed(e);
        victim->dev_cap = cap;
    }
    if (victim->staging_cap < n) {
        if (victim->staging) (void)hipHostFree(victim->staging);
        victim->staging = nullptr;
        victim->staging_cap = 0;
        const size_t cap = std::max<size_t>(n, 16384);
        e = hipHostMalloc(&victim->staging, cap, hipHostMallocDefault);
        if (e != hipSuccess) return hip_failed(e);
        victim->staging_cap = cap;
    }
    if (!victim->last_use) {
        e = hipEventCreateWithFlags(&victim->last_use, hipEventDisableTiming);
        if (e != hipSuccess) return hip_failed(e);
    }
    std::memcpy(victim->staging, bytes.data(), n);
    e = hipMemcpyAsync(victim->dev, victim->staging, n, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_failed(e);
    victim->bytes = bytes;
    victim->hash = h;
    *out = victim;
    return LEMA_OK;
}

lema_status release_table(DeviceState &d, TableEntry *t, hipStream_t stream) {
    hipError_t e = hipEventRecord(t->last_use, stream);
    if (e != hipSuccess) return hip_failed(e);
    t->last_stream = stream;
    t->recorded = true;
    t->stamp = ++d.clock;
    return LEMA_OK;
}

// Tile prefix sums and records of the non-empty segments.
struct TableBuild {
    std::vector<unsigned char> bytes;
    int nseg = 0;
    uint64_t total_tiles = 0;
};

void build_table(const std::vector<SegRec> &recs, TableBuild *tb) {
    const int n = static_cast<int>(recs.size());
    tb->nseg = n;
    tb->bytes.assign(table_bytes(n), 0);
    uint32_t *tile_begin = reinterpret_cast<uint32_t *>(tb->bytes.data());
    uint64_t tiles = 0;
    for (int i = 0; i < n; ++i) {
        tile_begin[i] = static_cast<uint32_t>(tiles);
        tiles += static_cast<uint64_t>((recs[i].numel + kTile - 1) / kTile);
    }
    tile_begin[n] = static_cast<uint32_t>(tiles);
    std::memcpy(tb->bytes.data() + table_tiles_bytes(n), recs.data(), sizeof(SegRec) * n);
    tb->total_tiles = tiles;
}

uint64_t count_tiles(const std::vector<SegRec> &recs) {
    uint64_t tiles = 0;
    for (const SegRec &r : recs) tiles += static_cast<uint64_t>((r.numel + kTile - 1) / kTile);
    return tiles;
}

}  // namespace

namespace {

// Launches are refused under stream capture: a captured graph would keep
// using a table the cache may later reuse.  Tables that travel in the kernel
// arguments are refused too, so that whether a call may be captured does
// not depend on its segment count.
lema_status refuse_capture(hipStream_t stream) {
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t ce = hipStreamIsCapturing(stream, &capture);
    if (ce != hipSuccess) return hip_failed(ce);
    return capture != hipStreamCaptureStatusNone ? LEMA_ERR_CAPTURE : LEMA_OK;
}

// An fp32 tile-kernel launch: a table of up to kInlineTableBytes goes in the
// kernel arguments, with no cache entry and no event; a larger one goes
// through the device cache.
lema_status launch_tile_table(
    const std::vector<unsigned char> &bytes, hipStream_t stream,
    const std::function<hipError_t(const void *, const InlineTable *)> &launch) {
    if (bytes.size() > kInlineTableBytes)
        return launch_on_table(bytes, stream,
                               [&](const void *table) { return launch(table, nullptr); });
    lema_status st = refuse_capture(stream);
    if (st != LEMA_OK) return st;
    InlineTable inl = {};
    std::memcpy(inl.w, bytes.data(), bytes.size());
    const hipError_t e = launch(nullptr, &inl);   // the arguments are copied at the launch
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

}  // namespace

lema_status launch_on_table(const std::vector<unsigned char> &bytes, hipStream_t stream,
                            const std::function<hipError_t(const void *)> &launch) {
    DeviceState *d = nullptr;
    lema_status st = device_state(&d, nullptr);
    if (st != LEMA_OK) return st;
    st = refuse_capture(stream);
    if (st != LEMA_OK) return st;
    std::lock_guard<std::mutex> lock(d->mu);
    TableEntry *t = nullptr;
    st = acquire_table(*d, bytes, stream, &t);
    if (st != LEMA_OK) return st;
    hipError_t e = launch(t->dev);
    lema_status rel = release_table(*d, t, stream);
    if (e != hipSuccess) return hip_failed(e);
    return rel;
}

// Workgroups of the AdamW step kernel allowed on one CU.  Each streams
// 7-12 KB of HBM traffic for its tile, from 5-12 arrays at once.  With every
// CU full of them (32 per CU) the HBM stacks see so many concurrent streams
// that they deliver 6-10% less than with 12 (measured on MI355X over 8-18
// per CU, for 28-38 B per parameter); the step that reads 8 resident
// micro-batches (48 B per parameter) does best at 9.
constexpr int kStepWorkgroupsPerCu = 12;
constexpr int kStepWorkgroupsPerCuManyMb = 9;
constexpr int kManyMicrobatches = 4;
// Launches of fewer tiles than this (under 64 rounds of 16 per CU over 256
// CUs) ramp up and drain for a larger share of their time and do better
// with 16 per CU: the rank-16 LoRA step (156 K tiles) 0.2214 against
// 0.2270 ms at 12, GPT-2 c_attn (13.8 K tiles) 21.84 against 22.20 us under
// the tracer (MI355X, interleaved runs on one box); the attention workload
// (1 M tiles) runs 2% slower at 16 than at 12.
constexpr int kStepWorkgroupsPerCuSmall = 16;
constexpr uint64_t kSmallLaunchTiles = uint64_t(1) << 18;

// LDS goes to a workgroup in whole granules: its static and dynamic LDS
// together, rounded up to a multiple of the granule.  On gfx950 the granule
// is 1280 bytes, 128 of them per CU (lema_probe_residency: 12,288 bytes per
// 64-lane workgroup let 12 share a CU, not 13; 16,384 let 9, 32,768 bytes
// per 256-lane workgroup 4), so only counts of the form floor(128 / k) are
// reachable through LDS: 12 or 14 per CU, never 13.
constexpr uint32_t kLdsGranule = 1280;

namespace {

// A small fixed cache of one number per kernel function (no allocation,
// so that lema_adamw_step_noalloc may use it); when full, values are
// computed again each time.
struct KernelCache {
    std::mutex mu;
    const void *fn[128] = {};
    int value[128] = {};
    int n = 0;
    template <class F>
    int get(const void *f, F compute) {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < n; ++i)
            if (fn[i] == f) return value[i];
        const int v = compute();
        if (n < 128) {
            fn[n] = f;
            value[n++] = v;
        }
        return v;
    }
};

// Static LDS of the kernels occupancy planning has asked about.
KernelCache g_static_lds;

uint32_t static_lds_bytes(const void *fn) {
    return static_cast<uint32_t>(g_static_lds.get(fn, [&] {
        hipFuncAttributes attr{};
        return hipFuncGetAttributes(&attr, fn) == hipSuccess ? int(attr.sharedSizeBytes) : 0;
    }));
}

// LDS of one workgroup (static plus dynamic) such that at most `per_cu`
// of them fit on one CU, as close to per_cu as the granule allows: the
// fewest granules k with floor(granules per CU / k) <= per_cu, at most
// 64 KiB.
uint32_t lds_per_workgroup(int lds_per_cu, int per_cu) {
    if (lds_per_cu <= 0 || per_cu <= 0) return 0;
    const uint32_t granules = static_cast<uint32_t>(lds_per_cu) / kLdsGranule;
    const uint32_t k = granules / static_cast<uint32_t>(per_cu + 1) + 1;
    return std::min<uint32_t>(k * kLdsGranule, 65536u);
}

// Workgroups of kernel `fn` that fit one CU by registers and static LDS
// alone (each kernel is always launched with the same workgroup size).
KernelCache g_occupancy;

}  // namespace

int compute_units() {
    DeviceState *d = nullptr;
    return device_state(&d, nullptr) == LEMA_OK ? d->cu_count : 0;
}

int register_occupancy(const void *fn, int lanes) {
    return g_occupancy.get(fn, [&] {
        int n = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, lanes, 0) == hipSuccess ? n : 0;
    });
}

uint32_t occupancy_lds_bytes(const void *fn, int workgroups_per_cu) {
    DeviceState *d = nullptr;
    if (fn == nullptr || device_state(&d, nullptr) != LEMA_OK) return 0;  // the launch reports it
    const uint32_t total = lds_per_workgroup(d->lds_per_cu, workgroups_per_cu);
    const uint32_t fixed = static_lds_bytes(fn);
    return total > fixed ? total - fixed : 0;
}

int step_workgroups_per_cu(int nmb, uint64_t tiles) {
    if (nmb >= kManyMicrobatches) return kStepWorkgroupsPerCuManyMb;
    return tiles < kSmallLaunchTiles ? kStepWorkgroupsPerCuSmall : kStepWorkgroupsPerCu;
}

uint32_t step_lds_bytes_for(GradMode grad_mode, bool with_delta, int nmb, uint64_t tiles) {
    return occupancy_lds_bytes(adamw_kernel_fn(grad_mode, with_delta, nmb),
                               step_workgroups_per_cu(nmb, tiles));
}

lema_status launch_adamw_recs(const std::vector<SegRec> &recs, const AdamwConsts &c,
                              GradMode grad_mode, hipStream_t stream) {
    if (recs.empty()) return LEMA_OK;
    if (count_tiles(recs) > kMaxTiles) return LEMA_ERR_SIZE;
    bool with_delta = false;
    for (const SegRec &r : recs) with_delta |= r.p[6] != 0;
    TableBuild tb;
    build_table(recs, &tb);
    const uint32_t lds = step_lds_bytes_for(grad_mode, with_delta, 0, tb.total_tiles);
    return launch_tile_table(tb.bytes, stream, [&](const void *table, const InlineTable *inl) {
        return launch_adamw(table, inl, tb.nseg, static_cast<uint32_t>(tb.total_tiles), grad_mode,
                            with_delta, c, stream, 0, lds);
    });
}

lema_status launch_adamw_sum_recs(std::vector<SegRec> recs, const std::vector<uint64_t> &lists,
                                  int nmb, const AdamwConsts &c, hipStream_t stream) {
    if (recs.empty()) return LEMA_OK;
    if (count_tiles(recs) > kMaxTiles) return LEMA_ERR_SIZE;
    bool with_delta = false;
    const int n = static_cast<int>(recs.size());
    for (int i = 0; i < n; ++i) {
        with_delta |= recs[i].p[6] != 0;
        recs[i].p[3] = table_bytes(n) + sizeof(uint64_t) * size_t(nmb) * size_t(i);
    }
    TableBuild tb;
    build_table(recs, &tb);
    const uint32_t lds = step_lds_bytes_for(kGradBf16Sum, with_delta, nmb, tb.total_tiles);
    tb.bytes.resize(table_bytes(n) + sizeof(uint64_t) * lists.size());
    std::memcpy(tb.bytes.data() + table_bytes(n), lists.data(), sizeof(uint64_t) * lists.size());
    return launch_tile_table(tb.bytes, stream, [&](const void *table, const InlineTable *inl) {
        return launch_adamw(table, inl, tb.nseg, static_cast<uint32_t>(tb.total_tiles),
                            kGradBf16Sum, with_delta, c, stream, nmb, lds);
    });
}

lema_status launch_accum_recs(const std::vector<SegRec> &recs, bool overwrite,
                              hipStream_t stream) {
    if (recs.empty()) return LEMA_OK;
    if (count_tiles(recs) > kMaxTiles) return LEMA_ERR_SIZE;
    TableBuild tb;
    build_table(recs, &tb);
    return launch_tile_table(tb.bytes, stream, [&](const void *table, const InlineTable *inl) {
        return launch_accum(table, inl, tb.nseg, static_cast<uint32_t>(tb.total_tiles), overwrite,
                            stream);
    });
}

lema_status launch_merge_recs(const std::vector<SegRec> &recs, hipStream_t stream) {
    if (recs.empty()) return LEMA_OK;
    if (count_tiles(recs) > kMaxTiles) return LEMA_ERR_SIZE;
    TableBuild tb;
    build_table(recs, &tb);
    return launch_tile_table(tb.bytes, stream, [&](const void *table, const InlineTable *inl) {
        return launch_merge(table, inl, tb.nseg, static_cast<uint32_t>(tb.total_tiles), stream);
    });
}

void adamw_records(const lema_adamw_seg *segs, int32_t nseg, std::vector<SegRec> *out,
                   const uint16_t *const *last_bf16) {
    out->clear();
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_seg &s = segs[i];
        if (s.numel == 0) continue;
        SegRec r{};
        r.p[0] = reinterpret_cast<uint64_t>(s.master);
        r.p[1] = reinterpret_cast<uint64_t>(s.exp_avg);
        r.p[2] = reinterpret_cast<uint64_t>(s.exp_avg_sq);
        r.p[3] = reinterpret_cast<uint64_t>(s.grad);
        r.p[4] = reinterpret_cast<uint64_t>(s.weight_bf16);
        r.p[5] = reinterpret_cast<uint64_t>(s.orig_bf16);
        r.p[6] = reinterpret_cast<uint64_t>(s.delta);
        r.p[7] = last_bf16 ? reinterpret_cast<uint64_t>(last_bf16[i]) : 0;
        r.numel = s.numel;
        out->push_back(r);
    }
}

}  // namespace lema

// ==================================================================== C ABI

using namespace lema;

extern "C" {

const char *lema_status_string(lema_status s) {
    switch (s) {
    case LEMA_OK: return "LEMA_OK";
    case LEMA_ERR_NULL: return "LEMA_ERR_NULL: required pointer is NULL or orig/delta unpaired";
    case LEMA_ERR_SIZE: return "LEMA_ERR_SIZE: negative or too large size";
    case LEMA_ERR_HPARAM: return "LEMA_ERR_HPARAM: hyperparameter or step out of range";
    case LEMA_ERR_DTYPE: return "LEMA_ERR_DTYPE: unknown gradient dtype";
    case LEMA_ERR_OVERLAP: return "LEMA_ERR_OVERLAP: arrays overlap where one is written";
    case LEMA_ERR_NOT_PINNED: return "LEMA_ERR_NOT_PINNED: host memory is not page-locked";
    case LEMA_ERR_HIP: return "LEMA_ERR_HIP: HIP runtime error (see lema_last_hip_error)";
    case LEMA_ERR_ALIGN: return "LEMA_ERR_ALIGN: pointer not aligned to its element size";
    case LEMA_ERR_CAPTURE: return "LEMA_ERR_CAPTURE: the stream is capturing a HIP graph";
    case LEMA_ERR_IO: return "LEMA_ERR_IO: checkpoint file unreadable, unwritable or malformed";
    case LEMA_ERR_NOT_FOUND: return "LEMA_ERR_NOT_FOUND: tensor not in the checkpoint file";
    default: return "unknown lema_status";
    }
}

int32_t lema_last_hip_error(void) { return t_last_hip_error; }

int32_t lema_version(void) { return 200; }   // 0.2.0: checkpoint files, reciprocal probe

lema_status lema_adamw_constants(const lema_adamw_args *args, lema_adamw_consts *out) {
    if (args == nullptr || out == nullptr) return LEMA_ERR_NULL;
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    const AdamwConsts c = derive_consts(args);
    out->beta1 = c.b1;
    out->one_minus_beta1 = c.omb1;
    out->beta2 = c.b2;
    out->one_minus_beta2 = c.omb2;
    out->eps = c.eps;
    out->decay = c.decay;
    out->step_size = c.step_size;
    out->inv_bias_correction2_root = c.inv_bc2_root;
    return LEMA_OK;
}

lema_status lema_adamw_step(const lema_adamw_seg *segs, int32_t nseg, const lema_adamw_args *args,
                            void *stream) {
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    std::vector<Span> spans;
    st = validate_adamw_segs(segs, nseg, args->grad_dtype, true, &spans);
    if (st != LEMA_OK) return st;
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    std::vector<SegRec> recs;
    adamw_records(segs, nseg, &recs, nullptr);
    return launch_adamw_recs(recs, derive_consts(args),
                             args->grad_dtype == LEMA_GRAD_FP32 ? kGradF32 : kGradBf16,
                             static_cast<hipStream_t>(stream));
}

lema_status lema_adamw_step_accum(const lema_adamw_seg *segs, const uint16_t *const *last_bf16,
                                  int32_t nseg, const lema_adamw_args *args, void *stream) {
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (args->grad_dtype != LEMA_GRAD_FP32) return LEMA_ERR_DTYPE;
    std::vector<Span> spans;
    st = validate_adamw_segs(segs, nseg, args->grad_dtype, true, &spans);
    if (st != LEMA_OK) return st;
    if (nseg > 0 && last_bf16 == nullptr) return LEMA_ERR_NULL;
    for (int32_t i = 0; i < nseg; ++i) {
        if (segs[i].numel == 0) continue;
        if (last_bf16[i] == nullptr) return LEMA_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(last_bf16[i]) & 1) return LEMA_ERR_ALIGN;
        add_span(spans, last_bf16[i], segs[i].numel, 2, false);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    std::vector<SegRec> recs;
    adamw_records(segs, nseg, &recs, last_bf16);
    return launch_adamw_recs(recs, derive_consts(args), kGradF32PlusBf16,
                             static_cast<hipStream_t>(stream));
}

lema_status lema_adamw_step_microbatches(const lema_adamw_seg *segs,
                                         const uint16_t *const *grads, int32_t nseg,
                                         int32_t nmb, const lema_adamw_args *args,
                                         void *stream) {
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (args->grad_dtype != LEMA_GRAD_BF16) return LEMA_ERR_DTYPE;
    if (nmb < 1 || nmb > kMaxMicrobatches) return LEMA_ERR_SIZE;
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && (segs == nullptr || grads == nullptr)) return LEMA_ERR_NULL;
    // validate as one-micro-batch segments on the first micro-batch, then
    // add the other micro-batches' spans
    std::vector<lema_adamw_seg> first(segs, segs + nseg);
    for (int32_t i = 0; i < nseg; ++i) {
        if (first[i].grad != nullptr) return LEMA_ERR_NULL;   // gradients come from `grads`
        first[i].grad = grads[size_t(i) * nmb];
    }
    std::vector<Span> spans;
    st = validate_adamw_segs(first.data(), nseg, LEMA_GRAD_BF16, true, &spans);
    if (st != LEMA_OK) return st;
    std::vector<SegRec> recs;
    std::vector<uint64_t> lists;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_seg &s = first[i];
        if (s.numel == 0) continue;
        uint64_t any = 0;
        for (int32_t j = 0; j < nmb; ++j) {
            const uint16_t *g = grads[size_t(i) * nmb + j];
            if (g == nullptr) return LEMA_ERR_NULL;
            if (reinterpret_cast<uintptr_t>(g) & 1) return LEMA_ERR_ALIGN;
            if (j > 0) add_span(spans, g, s.numel, 2, false);
            any |= reinterpret_cast<uint64_t>(g);
            lists.push_back(reinterpret_cast<uint64_t>(g));
        }
        SegRec r{};
        r.p[0] = reinterpret_cast<uint64_t>(s.master);
        r.p[1] = reinterpret_cast<uint64_t>(s.exp_avg);
        r.p[2] = reinterpret_cast<uint64_t>(s.exp_avg_sq);
        r.p[4] = reinterpret_cast<uint64_t>(s.weight_bf16);
        r.p[5] = reinterpret_cast<uint64_t>(s.orig_bf16);
        r.p[6] = reinterpret_cast<uint64_t>(s.delta);
        r.p[7] = any;
        r.numel = s.numel;
        r.reserved = nmb;
        recs.push_back(r);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    return launch_adamw_sum_recs(recs, lists, nmb, derive_consts(args),
                                 static_cast<hipStream_t>(stream));
}

lema_status lema_grad_accum(const lema_accum_seg *segs, int32_t nseg, int32_t overwrite,
                            void *stream) {
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    std::vector<Span> spans;
    std::vector<SegRec> recs;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_accum_seg &s = segs[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if (s.numel == 0) continue;
        if (!s.acc || !s.grad_bf16) return LEMA_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(s.acc) & 3) || (reinterpret_cast<uintptr_t>(s.grad_bf16) & 1))
            return LEMA_ERR_ALIGN;
        add_span(spans, s.acc, s.numel, 4, true);
        add_span(spans, s.grad_bf16, s.numel, 2, false);
        SegRec r{};
        r.p[0] = reinterpret_cast<uint64_t>(s.acc);
        r.p[1] = reinterpret_cast<uint64_t>(s.grad_bf16);
        r.numel = s.numel;
        recs.push_back(r);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    return launch_accum_recs(recs, overwrite != 0, static_cast<hipStream_t>(stream));
}

lema_status lema_merge_delta(const lema_merge_seg *segs, int32_t nseg, void *stream) {
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    std::vector<Span> spans;
    std::vector<SegRec> recs;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_merge_seg &s = segs[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if (s.numel == 0) continue;
        if (!s.base_bf16 || !s.delta || !s.merged_bf16) return LEMA_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(s.base_bf16) & 1) ||
            (reinterpret_cast<uintptr_t>(s.merged_bf16) & 1) ||
            (reinterpret_cast<uintptr_t>(s.delta) & 3))
            return LEMA_ERR_ALIGN;
        add_span(spans, s.base_bf16, s.numel, 2, false);
        add_span(spans, s.delta, s.numel, 4, false);
        add_span(spans, s.merged_bf16, s.numel, 2, true);
        SegRec r{};
        r.p[0] = reinterpret_cast<uint64_t>(s.base_bf16);
        r.p[1] = reinterpret_cast<uint64_t>(s.delta);
        r.p[2] = reinterpret_cast<uint64_t>(s.merged_bf16);
        r.numel = s.numel;
        recs.push_back(r);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    return launch_merge_recs(recs, static_cast<hipStream_t>(stream));
}

lema_status lema_host_alloc(void **out, size_t bytes) {
    if (out == nullptr) return LEMA_ERR_NULL;
    *out = nullptr;
    if (bytes == 0) return LEMA_ERR_SIZE;
    hipError_t e = hipHostMalloc(out, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        *out = nullptr;
        return hip_failed(e);
    }
    return LEMA_OK;
}

lema_status lema_host_free(void *p) {
    if (p == nullptr) return LEMA_OK;
    hipError_t e = hipHostFree(p);
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

// ------------------------------------------------ measurement aids

lema_status lema_measure_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (src == nullptr || dst == nullptr) return LEMA_ERR_NULL;
    if (bytes == 0 || (bytes % 16) != 0) return LEMA_ERR_SIZE;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0)
        return LEMA_ERR_ALIGN;
    std::vector<Span> spans;
    add_span(spans, src, static_cast<int64_t>(bytes), 1, false);
    add_span(spans, dst, static_cast<int64_t>(bytes), 1, true);
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    hipError_t e = launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

lema_status lema_probe_fp32(const float *a, const float *b, float *quot, float *root,
                            uint16_t *bf16, int64_t n, void *stream) {
    if (n < 0) return LEMA_ERR_SIZE;
    if (n == 0) return LEMA_OK;
    if (!a || !b || !quot || !root || !bf16) return LEMA_ERR_NULL;
    hipError_t e = launch_fp32_probe(a, b, quot, root, bf16, n, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

lema_status lema_table_cache_stats(int64_t out[4]) {
    if (out == nullptr) return LEMA_ERR_NULL;
    DeviceState *d = nullptr;
    lema_status st = device_state(&d, nullptr);
    if (st != LEMA_OK) return st;
    std::lock_guard<std::mutex> lock(d->mu);
    out[0] = d->hits;
    out[1] = d->uploads;
    out[2] = d->waits;
    out[3] = static_cast<int64_t>(d->entries.size());
    return LEMA_OK;
}

lema_status lema_step_lds_reservation(int32_t microbatches, int32_t *lds_per_cu,
                                      int32_t *reserved_bytes) {
    if (lds_per_cu == nullptr || reserved_bytes == nullptr) return LEMA_ERR_NULL;
    if (microbatches < 0) return LEMA_ERR_SIZE;
    DeviceState *d = nullptr;
    lema_status st = device_state(&d, nullptr);
    if (st != LEMA_OK) return st;
    *lds_per_cu = d->lds_per_cu;
    *reserved_bytes = static_cast<int32_t>(
        microbatches >= 1 && microbatches <= kMaxMicrobatches
            ? step_lds_bytes_for(kGradBf16Sum, true, microbatches, kSmallLaunchTiles)
            : step_lds_bytes_for(kGradBf16, true, 0, kSmallLaunchTiles));
    return LEMA_OK;
}

lema_status lema_probe_residency(uint64_t *records, int32_t workgroups, int32_t lanes,
                                 int32_t lds_bytes, int32_t spin_us, void *stream) {
    if (records == nullptr) return LEMA_ERR_NULL;
    if (workgroups < 1 || workgroups > (1 << 20) || lanes < 64 || lanes > 1024 || lanes % 64 ||
        lds_bytes < 0 || lds_bytes > 65536 || spin_us < 1 || spin_us > 1000)
        return LEMA_ERR_SIZE;
    if (reinterpret_cast<uintptr_t>(records) & 7) return LEMA_ERR_ALIGN;
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return hip_failed(e);
    const uint64_t ticks = std::max<uint64_t>(1, uint64_t(khz) * uint64_t(spin_us) / 1000);
    e = launch_residency_probe(records, workgroups, lanes, static_cast<uint32_t>(lds_bytes), ticks,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

lema_status lema_step_occupancy(int32_t kernel, int32_t out[6]) {
    if (out == nullptr) return LEMA_ERR_NULL;
    const void *fn = nullptr;
    int lanes = kBlock, per_cu = 0;
    switch (kernel) {
    case 0:
        fn = adamw_kernel_fn(kGradBf16, true, 0);
        per_cu = step_workgroups_per_cu(0, kSmallLaunchTiles);
        break;
    case 1:
        fn = adamw_kernel_fn(kGradBf16Sum, true, 8);
        per_cu = step_workgroups_per_cu(8, kSmallLaunchTiles);
        break;
    case 3:
        fn = adamw_kernel_fn(kGradBf16, true, 0);
        per_cu = step_workgroups_per_cu(0, 0);
        break;
    case 2:
        fn = adamw_q8_kernel_fn(true, kQGradBf16, true, kQBlock, kQRowsWave);
        lanes = kQBlock;
        per_cu = kQ8StepWorkgroupsPerCu;
        break;
    default: return LEMA_ERR_SIZE;
    }
    hipFuncAttributes attr{};
    hipError_t e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess) return hip_failed(e);
    int by_regs = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&by_regs, fn, lanes, 0);
    if (e != hipSuccess) return hip_failed(e);
    out[0] = lanes;
    out[1] = static_cast<int32_t>(attr.sharedSizeBytes);
    out[2] = static_cast<int32_t>(occupancy_lds_bytes(fn, per_cu));
    out[3] = per_cu;
    out[4] = by_regs;
    out[5] = static_cast<int32_t>(kLdsGranule);
    return LEMA_OK;
}

lema_status lema_device_info(int32_t *compute_units, int32_t *tile_elements) {
    if (compute_units == nullptr || tile_elements == nullptr) return LEMA_ERR_NULL;
    DeviceState *d = nullptr;
    lema_status st = device_state(&d, nullptr);
    if (st != LEMA_OK) return st;
    *compute_units = d->cu_count;
    *tile_elements = static_cast<int32_t>(kTile);
    return LEMA_OK;
}

}  // extern "C"
