// lema_slot.cpp -- slot-pool streaming of host-resident optimizer state.
//
// LEMA README: "TensorStore: Unified Streaming Core" streams optimizer states
// through a slot-pool address space; "Selective Full Fine-Tuning" keeps the
// fp32 states in (pinned) host RAM; "Features" describes async prefetch from
// pinned RAM to VRAM hiding the PCIe latency.  Here the pool is two (or more)
// HBM slots on one copy stream and one compute stream:
//
//   copy stream   : H2D(0) H2D(1) D2H(0) H2D(2) D2H(1) ... H2D(L-1) D2H(L-2) D2H(L-1)
//   compute stream:        K(0)   K(1)          K(2)   ...          K(L-1)
//
// K(i) waits for H2D(i); D2H(i) waits for K(i).  Slot i mod nslots is
// rewritten by H2D(i) only after D2H(i - nslots), which precedes it on the
// copy stream, so no slot is overwritten while still in use.  The host
// enqueues everything without waiting and synchronizes once at the end.
//
// With a separate write-back stream (lema_slot_pool_set_writeback_stream)
// the D2H copies move there, so the two PCIe directions run at once:
//
//   copy stream     : H2D(0) H2D(1) H2D(2) ...      (H2D(i) waits for D2H(i - nslots))
//   write-back      :        D2H(0) D2H(1) ...      (D2H(i) waits for K(i))
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <mutex>
#include <thread>
#include <utility>
#include <vector>

#include "lema.h"
#include "lema_host_internal.h"
#include "lema_internal.h"

using namespace lema;

struct lema_slot_pool {
    int device = 0;
    char *base = nullptr;
    size_t slot_bytes = 0;
    int nslots = 0;
    hipStream_t copy = nullptr;
    hipStream_t compute = nullptr;
    hipStream_t writeback = nullptr;  // NULL: D2H copies share the copy stream
    std::vector<hipEvent_t> events;   // 6 per layer, grown on demand, reused
    char *staging[2] = {nullptr, nullptr};   // page-locked, slot_bytes each (staged path)
    std::mutex mu;
};

namespace {

constexpr size_t kSlotAlign = 256;

size_t align_up(size_t x) { return (x + kSlotAlign - 1) & ~(kSlotAlign - 1); }

// Bytes one layer needs in a slot: master, m, v, grad (bf16), weight (bf16)
// per segment, each array starting on a 256-byte boundary.
size_t layer_slot_bytes(const lema_layer &L) {
    size_t off = 0;
    for (int32_t i = 0; i < L.nseg; ++i) {
        const size_t n = static_cast<size_t>(L.host_segs[i].numel);
        if (n == 0) continue;
        off = align_up(off) + 4 * n;
        off = align_up(off) + 4 * n;
        off = align_up(off) + 4 * n;
        off = align_up(off) + 2 * n;
        off = align_up(off) + 2 * n;
    }
    return off;
}

// Device-side segment descriptors of layer L placed at `slot`.
void slot_segments(const lema_layer &L, char *slot, std::vector<lema_adamw_seg> *out) {
    out->clear();
    size_t off = 0;
    for (int32_t i = 0; i < L.nseg; ++i) {
        const lema_adamw_seg &h = L.host_segs[i];
        const size_t n = static_cast<size_t>(h.numel);
        if (n == 0) continue;
        lema_adamw_seg d{};
        off = align_up(off); d.master = reinterpret_cast<float *>(slot + off); off += 4 * n;
        off = align_up(off); d.exp_avg = reinterpret_cast<float *>(slot + off); off += 4 * n;
        off = align_up(off); d.exp_avg_sq = reinterpret_cast<float *>(slot + off); off += 4 * n;
        off = align_up(off); d.grad = slot + off; off += 2 * n;
        off = align_up(off); d.weight_bf16 = reinterpret_cast<uint16_t *>(slot + off); off += 2 * n;
        d.numel = h.numel;
        out->push_back(d);
    }
}

// True if [p, p + bytes) lies in page-locked host memory known to HIP.
bool is_pinned(const void *p, size_t bytes) {
    hipPointerAttribute_t attr{};
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // a pageable pointer is an answer, not an error
        return false;
    }
    if (attr.type != hipMemoryTypeHost) return false;
    uintptr_t start = 0;
    size_t size = 0;
    if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR,
                               reinterpret_cast<hipDeviceptr_t>(const_cast<void *>(p))) == hipSuccess &&
        hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE,
                               reinterpret_cast<hipDeviceptr_t>(const_cast<void *>(p))) == hipSuccess &&
        size != 0) {
        return reinterpret_cast<uintptr_t>(p) + bytes <= start + size;
    }
    (void)hipGetLastError();
    return true;
}

lema_status ensure_events(lema_slot_pool *pool, size_t n) {
    while (pool->events.size() < n) {
        hipEvent_t ev;
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_failed(e);
        pool->events.push_back(ev);
    }
    return LEMA_OK;
}

enum { EV_H2D_BEGIN = 0, EV_H2D_END, EV_K_BEGIN, EV_K_END, EV_D2H_BEGIN, EV_D2H_END, EV_PER_LAYER };

// The non-empty segments of a layer, in order.
void nonempty_segments(const lema_layer &L, std::vector<lema_adamw_seg> *out) {
    out->clear();
    for (int32_t i = 0; i < L.nseg; ++i)
        if (L.host_segs[i].numel > 0) out->push_back(L.host_segs[i]);
}

// Host -> slot copies of master, m, v and the bf16 gradient (14 B/param).
hipError_t enqueue_upload(const std::vector<lema_adamw_seg> &src,
                          const std::vector<lema_adamw_seg> &dst, hipStream_t s, double *bytes) {
    hipError_t e = hipSuccess;
    for (size_t k = 0; k < src.size() && e == hipSuccess; ++k) {
        const size_t n = size_t(src[k].numel);
        e = hipMemcpyAsync(dst[k].master, src[k].master, 4 * n, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipMemcpyAsync(dst[k].exp_avg, src[k].exp_avg, 4 * n, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipMemcpyAsync(dst[k].exp_avg_sq, src[k].exp_avg_sq, 4 * n, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipMemcpyAsync(const_cast<void *>(dst[k].grad), src[k].grad, 2 * n, hipMemcpyHostToDevice, s);
        *bytes += 14.0 * double(n);
    }
    return e;
}

// Slot -> host copies of master, m, v and the bf16 weight (14 B/param).
hipError_t enqueue_writeback(const std::vector<lema_adamw_seg> &src,
                             const std::vector<lema_adamw_seg> &dst, hipStream_t s, double *bytes) {
    hipError_t e = hipSuccess;
    for (size_t k = 0; k < src.size() && e == hipSuccess; ++k) {
        const size_t n = size_t(src[k].numel);
        e = hipMemcpyAsync(dst[k].master, src[k].master, 4 * n, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipMemcpyAsync(dst[k].exp_avg, src[k].exp_avg, 4 * n, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipMemcpyAsync(dst[k].exp_avg_sq, src[k].exp_avg_sq, 4 * n, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipMemcpyAsync(dst[k].weight_bf16, src[k].weight_bf16, 2 * n, hipMemcpyDeviceToHost, s);
        *bytes += 14.0 * double(n);
    }
    return e;
}

// Copy intervals from the pool's events: per-direction sums, their union,
// kernel time, and the span from the first upload to the last write-back.
void fill_stats(lema_slot_pool *pool, int32_t nlayers, double h2d_bytes, double d2h_bytes,
                lema_stream_stats *out) {
    auto ev = [&](int layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    lema_stream_stats s{};
    s.h2d_bytes = h2d_bytes;
    s.d2h_bytes = d2h_bytes;
    std::vector<std::pair<float, float>> busy;
    const hipEvent_t t0 = ev(0, EV_H2D_BEGIN);
    float ms = 0.f, b = 0.f, en = 0.f;
    for (int32_t i = 0; i < nlayers; ++i) {
        if (hipEventElapsedTime(&b, t0, ev(i, EV_H2D_BEGIN)) == hipSuccess &&
            hipEventElapsedTime(&en, t0, ev(i, EV_H2D_END)) == hipSuccess) {
            s.h2d_ms += en - b;
            busy.emplace_back(b, en);
        }
        if (hipEventElapsedTime(&b, t0, ev(i, EV_D2H_BEGIN)) == hipSuccess &&
            hipEventElapsedTime(&en, t0, ev(i, EV_D2H_END)) == hipSuccess) {
            s.d2h_ms += en - b;
            busy.emplace_back(b, en);
        }
        if (hipEventElapsedTime(&ms, ev(i, EV_K_BEGIN), ev(i, EV_K_END)) == hipSuccess) {
            s.kernel_ms += ms;
            if (i == nlayers - 1) s.last_kernel_ms = ms;
        }
    }
    std::sort(busy.begin(), busy.end());
    float lo = 0.f, hi = -1.f;
    for (const auto &iv : busy) {
        if (iv.first > hi) {
            if (hi > lo) s.copy_busy_ms += hi - lo;
            lo = iv.first;
            hi = iv.second;
        } else if (iv.second > hi) {
            hi = iv.second;
        }
    }
    if (hi > lo) s.copy_busy_ms += hi - lo;
    if (hipEventElapsedTime(&ms, t0, ev(nlayers - 1, EV_D2H_END)) == hipSuccess) s.wall_ms = ms;
    *out = s;
}

// ---------------------------------------------------- staged host copies

struct CopyItem {
    void *dst;
    const void *src;
    size_t bytes;
};

// memcpy of a list of ranges split evenly over `threads` host threads.
void parallel_copy(const std::vector<CopyItem> &items, int threads) {
    size_t total = 0;
    for (const CopyItem &c : items) total += c.bytes;
    if (threads <= 1 || total < (size_t(8) << 20)) {
        for (const CopyItem &c : items) std::memcpy(c.dst, c.src, c.bytes);
        return;
    }
    const size_t share = ((total + threads - 1) / threads + 63) & ~size_t(63);
    auto run = [&](size_t begin, size_t end) {
        size_t pos = 0;
        for (const CopyItem &c : items) {
            const size_t lo = std::max(begin, pos), hi = std::min(end, pos + c.bytes);
            if (lo < hi)
                std::memcpy(static_cast<char *>(c.dst) + (lo - pos),
                            static_cast<const char *>(c.src) + (lo - pos), hi - lo);
            pos += c.bytes;
            if (pos >= end) break;
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < threads; ++t) {
        const size_t b = size_t(t) * share;
        if (b >= total) break;
        pool.emplace_back(run, b, std::min(total, b + share));
    }
    run(0, std::min(total, share));
    for (std::thread &t : pool) t.join();
}

// Items moving a layer's inputs (master, m, v, grad) from the caller's memory
// into staging laid out like the slot, or its outputs (master, m, v, weight)
// back from staging.
void staging_items(const std::vector<lema_adamw_seg> &host, const std::vector<lema_adamw_seg> &stage,
                   bool inbound, std::vector<CopyItem> *out) {
    out->clear();
    for (size_t k = 0; k < host.size(); ++k) {
        const size_t n = size_t(host[k].numel);
        if (inbound) {
            out->push_back({stage[k].master, host[k].master, 4 * n});
            out->push_back({stage[k].exp_avg, host[k].exp_avg, 4 * n});
            out->push_back({stage[k].exp_avg_sq, host[k].exp_avg_sq, 4 * n});
            out->push_back({const_cast<void *>(stage[k].grad), host[k].grad, 2 * n});
        } else {
            out->push_back({host[k].master, stage[k].master, 4 * n});
            out->push_back({host[k].exp_avg, stage[k].exp_avg, 4 * n});
            out->push_back({host[k].exp_avg_sq, stage[k].exp_avg_sq, 4 * n});
            out->push_back({host[k].weight_bf16, stage[k].weight_bf16, 2 * n});
        }
    }
}

lema_status validate_layers(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                            const lema_adamw_args *args, std::vector<Span> *spans) {
    if (pool == nullptr) return LEMA_ERR_NULL;
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (args->grad_dtype != LEMA_GRAD_BF16) return LEMA_ERR_DTYPE;
    if (nlayers < 0) return LEMA_ERR_SIZE;
    if (nlayers > 0 && layers == nullptr) return LEMA_ERR_NULL;
    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer &L = layers[i];
        st = validate_adamw_segs(L.host_segs, L.nseg, LEMA_GRAD_BF16, false, spans);
        if (st != LEMA_OK) return st;
        if (layer_slot_bytes(L) > pool->slot_bytes) return LEMA_ERR_SIZE;
    }
    if (any_conflict(*spans)) return LEMA_ERR_OVERLAP;
    return LEMA_OK;
}

}  // namespace

extern "C" {

lema_status lema_slot_pool_create(void *device_base, size_t slot_bytes, int32_t nslots,
                                  void *copy_stream, void *compute_stream, lema_slot_pool **out) {
    if (out == nullptr || device_base == nullptr) return LEMA_ERR_NULL;
    *out = nullptr;
    if (nslots < 2 || slot_bytes == 0 || (slot_bytes % kSlotAlign) != 0) return LEMA_ERR_SIZE;
    if (copy_stream == compute_stream) return LEMA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(device_base) % kSlotAlign) != 0) return LEMA_ERR_ALIGN;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    lema_slot_pool *p = new (std::nothrow) lema_slot_pool;
    if (p == nullptr) return LEMA_ERR_SIZE;
    p->device = dev;
    p->base = static_cast<char *>(device_base);
    p->slot_bytes = slot_bytes;
    p->nslots = nslots;
    p->copy = static_cast<hipStream_t>(copy_stream);
    p->compute = static_cast<hipStream_t>(compute_stream);
    *out = p;
    return LEMA_OK;
}

lema_status lema_slot_pool_set_writeback_stream(lema_slot_pool *pool, void *stream) {
    if (pool == nullptr) return LEMA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (s != nullptr && (s == pool->copy || s == pool->compute)) return LEMA_ERR_NULL;
    std::lock_guard<std::mutex> lock(pool->mu);
    pool->writeback = s;
    return LEMA_OK;
}

lema_status lema_slot_pool_destroy(lema_slot_pool *pool) {
    if (pool == nullptr) return LEMA_OK;
    lema_status st = LEMA_OK;
    {
        std::lock_guard<std::mutex> lock(pool->mu);
        for (hipEvent_t ev : pool->events) {
            hipError_t e = hipEventSynchronize(ev);
            if (e != hipSuccess && e != hipErrorInvalidResourceHandle && st == LEMA_OK) st = hip_failed(e);
            (void)hipEventDestroy(ev);
        }
        pool->events.clear();
        for (char *&p : pool->staging) {
            if (p) (void)hipHostFree(p);
            p = nullptr;
        }
    }
    delete pool;
    return st;
}

lema_status lema_slot_stream(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                             const lema_adamw_args *args, lema_stream_stats *stats) {
    // ---- validation of every layer before anything is enqueued
    std::vector<Span> spans;
    lema_status st = validate_layers(pool, layers, nlayers, args, &spans);
    if (st != LEMA_OK) return st;
    for (const Span &s : spans)
        if (s.hi > s.lo && !is_pinned(reinterpret_cast<const void *>(s.lo), s.hi - s.lo))
            return LEMA_ERR_NOT_PINNED;
    if (nlayers == 0) {
        if (stats) *stats = lema_stream_stats{};
        return LEMA_OK;
    }
    const auto call_start = std::chrono::steady_clock::now();

    std::lock_guard<std::mutex> lock(pool->mu);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_failed(e);
    if (cur != pool->device) return LEMA_ERR_HIP;
    st = ensure_events(pool, size_t(nlayers) * EV_PER_LAYER);
    if (st != LEMA_OK) return st;

    const AdamwConsts consts = derive_consts(args);
    auto ev = [&](int layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    std::vector<std::vector<lema_adamw_seg>> dev_segs(nlayers), host_segs(nlayers);
    double h2d_bytes = 0, d2h_bytes = 0;
    hipStream_t d2h_stream = pool->writeback ? pool->writeback : pool->copy;

    auto copy_back = [&](int j) -> lema_status {
        hipError_t err = hipStreamWaitEvent(d2h_stream, ev(j, EV_K_END), 0);
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_BEGIN), d2h_stream);
        if (err == hipSuccess) err = enqueue_writeback(dev_segs[j], host_segs[j], d2h_stream, &d2h_bytes);
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_END), d2h_stream);
        return err == hipSuccess ? LEMA_OK : hip_failed(err);
    };

    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer &L = layers[i];
        char *slot = pool->base + size_t(i % pool->nslots) * pool->slot_bytes;
        slot_segments(L, slot, &dev_segs[i]);
        nonempty_segments(L, &host_segs[i]);

        // host -> slot; with a separate write-back stream the slot must first
        // have been copied back from its previous occupant
        e = hipSuccess;
        if (pool->writeback && i >= pool->nslots)
            e = hipStreamWaitEvent(pool->copy, ev(i - pool->nslots, EV_D2H_END), 0);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_H2D_BEGIN), pool->copy);
        if (e == hipSuccess) e = enqueue_upload(host_segs[i], dev_segs[i], pool->copy, &h2d_bytes);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_H2D_END), pool->copy);
        if (e != hipSuccess) return hip_failed(e);

        // the step on the slot
        e = hipStreamWaitEvent(pool->compute, ev(i, EV_H2D_END), 0);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_K_BEGIN), pool->compute);
        if (e != hipSuccess) return hip_failed(e);
        std::vector<SegRec> recs;
        adamw_records(dev_segs[i].data(), int32_t(dev_segs[i].size()), &recs, nullptr);
        st = launch_adamw_recs(recs, consts, kGradBf16, pool->compute);
        if (st != LEMA_OK) return st;
        e = hipEventRecord(ev(i, EV_K_END), pool->compute);
        if (e != hipSuccess) return hip_failed(e);

        // slot -> host for the previous layer, behind this layer's upload
        if (i >= 1) {
            st = copy_back(i - 1);
            if (st != LEMA_OK) return st;
        }
    }
    st = copy_back(nlayers - 1);
    if (st != LEMA_OK) return st;
    e = hipEventSynchronize(ev(nlayers - 1, EV_D2H_END));
    if (e != hipSuccess) return hip_failed(e);

    if (stats) {
        fill_stats(pool, nlayers, h2d_bytes, d2h_bytes, stats);
        stats->call_ms = std::chrono::duration<double, std::milli>(
                             std::chrono::steady_clock::now() - call_start).count();
    }
    return LEMA_OK;
}

lema_status lema_slot_stream_staged(lema_slot_pool *pool, const lema_layer *layers,
                                    int32_t nlayers, const lema_adamw_args *args,
                                    int32_t host_threads, lema_stream_stats *stats) {
    std::vector<Span> spans;
    lema_status st = validate_layers(pool, layers, nlayers, args, &spans);
    if (st != LEMA_OK) return st;
    if (host_threads < 0 || host_threads > 256) return LEMA_ERR_SIZE;
    if (nlayers == 0) {
        if (stats) *stats = lema_stream_stats{};
        return LEMA_OK;
    }
    int threads = host_threads;
    if (threads == 0) {
        const unsigned hc = std::thread::hardware_concurrency();
        threads = int(std::min(16u, hc == 0 ? 4u : hc));
    }
    const auto call_start = std::chrono::steady_clock::now();

    std::lock_guard<std::mutex> lock(pool->mu);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_failed(e);
    if (cur != pool->device) return LEMA_ERR_HIP;
    for (int b = 0; b < 2; ++b) {
        if (pool->staging[b] == nullptr) {
            e = hipHostMalloc(reinterpret_cast<void **>(&pool->staging[b]), pool->slot_bytes,
                              hipHostMallocDefault);
            if (e != hipSuccess) {
                pool->staging[b] = nullptr;
                return hip_failed(e);
            }
        }
    }
    st = ensure_events(pool, size_t(nlayers) * EV_PER_LAYER);
    if (st != LEMA_OK) return st;

    const AdamwConsts consts = derive_consts(args);
    auto ev = [&](int layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    std::vector<std::vector<lema_adamw_seg>> dev_segs(nlayers), stage_segs(nlayers),
        host_segs(nlayers);
    double h2d_bytes = 0, d2h_bytes = 0, in_ms = 0, out_ms = 0;
    hipStream_t d2h_stream = pool->writeback ? pool->writeback : pool->copy;
    std::vector<CopyItem> items;
    using clock = std::chrono::steady_clock;

    // Layer i goes caller memory -> staging[i % 2] -> slot[i % 2] -> staging[i % 2]
    // -> caller memory.  Layer i + 2 reuses both only after the host has
    // copied layer i out of staging, which itself waited for its write-back.
    auto stage_in_and_enqueue = [&](int i) -> lema_status {
        const lema_layer &L = layers[i];
        const int b = i % 2;
        slot_segments(L, pool->base + size_t(b) * pool->slot_bytes, &dev_segs[i]);
        slot_segments(L, pool->staging[b], &stage_segs[i]);
        nonempty_segments(L, &host_segs[i]);
        staging_items(host_segs[i], stage_segs[i], true, &items);
        const auto t0 = clock::now();
        parallel_copy(items, threads);
        in_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();

        hipError_t err = hipEventRecord(ev(i, EV_H2D_BEGIN), pool->copy);
        if (err == hipSuccess) err = enqueue_upload(stage_segs[i], dev_segs[i], pool->copy, &h2d_bytes);
        if (err == hipSuccess) err = hipEventRecord(ev(i, EV_H2D_END), pool->copy);
        if (err == hipSuccess) err = hipStreamWaitEvent(pool->compute, ev(i, EV_H2D_END), 0);
        if (err == hipSuccess) err = hipEventRecord(ev(i, EV_K_BEGIN), pool->compute);
        if (err != hipSuccess) return hip_failed(err);
        std::vector<SegRec> recs;
        adamw_records(dev_segs[i].data(), int32_t(dev_segs[i].size()), &recs, nullptr);
        lema_status s2 = launch_adamw_recs(recs, consts, kGradBf16, pool->compute);
        if (s2 != LEMA_OK) return s2;
        err = hipEventRecord(ev(i, EV_K_END), pool->compute);
        if (err == hipSuccess) err = hipStreamWaitEvent(d2h_stream, ev(i, EV_K_END), 0);
        if (err == hipSuccess) err = hipEventRecord(ev(i, EV_D2H_BEGIN), d2h_stream);
        if (err == hipSuccess) err = enqueue_writeback(dev_segs[i], stage_segs[i], d2h_stream, &d2h_bytes);
        if (err == hipSuccess) err = hipEventRecord(ev(i, EV_D2H_END), d2h_stream);
        return err == hipSuccess ? LEMA_OK : hip_failed(err);
    };
    auto wait_and_stage_out = [&](int i) -> lema_status {
        hipError_t err = hipEventSynchronize(ev(i, EV_D2H_END));
        if (err != hipSuccess) return hip_failed(err);
        staging_items(host_segs[i], stage_segs[i], false, &items);
        const auto t0 = clock::now();
        parallel_copy(items, threads);
        out_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
        return LEMA_OK;
    };

    for (int i = 0; i < std::min(nlayers, 2); ++i) {
        st = stage_in_and_enqueue(i);
        if (st != LEMA_OK) return st;
    }
    for (int i = 0; i < nlayers; ++i) {
        st = wait_and_stage_out(i);
        if (st != LEMA_OK) return st;
        if (i + 2 < nlayers) {
            st = stage_in_and_enqueue(i + 2);
            if (st != LEMA_OK) return st;
        }
    }

    if (stats) {
        fill_stats(pool, nlayers, h2d_bytes, d2h_bytes, stats);
        stats->host_in_ms = in_ms;
        stats->host_out_ms = out_ms;
        stats->call_ms = std::chrono::duration<double, std::milli>(clock::now() - call_start).count();
    }
    return LEMA_OK;
}

}  // extern "C"
