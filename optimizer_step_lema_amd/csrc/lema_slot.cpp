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
#include <mutex>
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
    }
    delete pool;
    return st;
}

lema_status lema_slot_stream(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                             const lema_adamw_args *args, lema_stream_stats *stats) {
    if (pool == nullptr) return LEMA_ERR_NULL;
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (args->grad_dtype != LEMA_GRAD_BF16) return LEMA_ERR_DTYPE;
    if (nlayers < 0) return LEMA_ERR_SIZE;
    if (nlayers > 0 && layers == nullptr) return LEMA_ERR_NULL;

    // ---- validation of every layer before anything is enqueued
    std::vector<Span> spans;
    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer &L = layers[i];
        st = validate_adamw_segs(L.host_segs, L.nseg, LEMA_GRAD_BF16, false, &spans);
        if (st != LEMA_OK) return st;
        if (layer_slot_bytes(L) > pool->slot_bytes) return LEMA_ERR_SIZE;
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    for (const Span &s : spans)
        if (s.hi > s.lo && !is_pinned(reinterpret_cast<const void *>(s.lo), s.hi - s.lo))
            return LEMA_ERR_NOT_PINNED;
    if (nlayers == 0) {
        if (stats) *stats = lema_stream_stats{};
        return LEMA_OK;
    }

    std::lock_guard<std::mutex> lock(pool->mu);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_failed(e);
    if (cur != pool->device) return LEMA_ERR_HIP;
    st = ensure_events(pool, size_t(nlayers) * EV_PER_LAYER);
    if (st != LEMA_OK) return st;

    const AdamwConsts consts = derive_consts(args);
    auto ev = [&](int layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    std::vector<std::vector<lema_adamw_seg>> dev_segs(nlayers);
    double h2d_bytes = 0, d2h_bytes = 0;

    hipStream_t d2h_stream = pool->writeback ? pool->writeback : pool->copy;
    auto copy_back = [&](int j) -> lema_status {
        const lema_layer &L = layers[j];
        hipError_t err = hipStreamWaitEvent(d2h_stream, ev(j, EV_K_END), 0);
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_BEGIN), d2h_stream);
        size_t k = 0;
        for (int32_t s = 0; s < L.nseg && err == hipSuccess; ++s) {
            const lema_adamw_seg &h = L.host_segs[s];
            if (h.numel == 0) continue;
            const lema_adamw_seg &d = dev_segs[j][k++];
            const size_t n = size_t(h.numel);
            err = hipMemcpyAsync(h.master, d.master, 4 * n, hipMemcpyDeviceToHost, d2h_stream);
            if (err == hipSuccess) err = hipMemcpyAsync(h.exp_avg, d.exp_avg, 4 * n, hipMemcpyDeviceToHost, d2h_stream);
            if (err == hipSuccess) err = hipMemcpyAsync(h.exp_avg_sq, d.exp_avg_sq, 4 * n, hipMemcpyDeviceToHost, d2h_stream);
            if (err == hipSuccess) err = hipMemcpyAsync(h.weight_bf16, d.weight_bf16, 2 * n, hipMemcpyDeviceToHost, d2h_stream);
            d2h_bytes += 14.0 * double(n);
        }
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_END), d2h_stream);
        return err == hipSuccess ? LEMA_OK : hip_failed(err);
    };

    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer &L = layers[i];
        char *slot = pool->base + size_t(i % pool->nslots) * pool->slot_bytes;
        slot_segments(L, slot, &dev_segs[i]);

        // host -> slot; with a separate write-back stream the slot must first
        // have been copied back from its previous occupant
        e = hipSuccess;
        if (pool->writeback && i >= pool->nslots)
            e = hipStreamWaitEvent(pool->copy, ev(i - pool->nslots, EV_D2H_END), 0);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_H2D_BEGIN), pool->copy);
        size_t k = 0;
        for (int32_t s = 0; s < L.nseg && e == hipSuccess; ++s) {
            const lema_adamw_seg &h = L.host_segs[s];
            if (h.numel == 0) continue;
            const lema_adamw_seg &d = dev_segs[i][k++];
            const size_t n = size_t(h.numel);
            e = hipMemcpyAsync(d.master, h.master, 4 * n, hipMemcpyHostToDevice, pool->copy);
            if (e == hipSuccess) e = hipMemcpyAsync(d.exp_avg, h.exp_avg, 4 * n, hipMemcpyHostToDevice, pool->copy);
            if (e == hipSuccess) e = hipMemcpyAsync(d.exp_avg_sq, h.exp_avg_sq, 4 * n, hipMemcpyHostToDevice, pool->copy);
            if (e == hipSuccess) e = hipMemcpyAsync(const_cast<void *>(d.grad), h.grad, 2 * n, hipMemcpyHostToDevice, pool->copy);
            h2d_bytes += 14.0 * double(n);
        }
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
        lema_stream_stats s{};
        s.h2d_bytes = h2d_bytes;
        s.d2h_bytes = d2h_bytes;
        // copy intervals relative to the first upload, then their union
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
        *stats = s;
    }
    return LEMA_OK;
}

}  // extern "C"
