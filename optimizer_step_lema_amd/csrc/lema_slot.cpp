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
//
// Both pipelines work on a layer plan: the list of the layer's arrays, each
// with its host address, its offset in the slot and whether it is copied in,
// out or both, plus the launch of the layer's step on the slot.  fp32 state
// (lema_slot_stream*) and int8 state with row scales (lema_slot_stream_q8,
// README "Quantization": host memory holds the codes and scales) differ
// only in their plans.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <functional>
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
    std::vector<hipEvent_t> events;   // grown on demand, reused by later calls
    std::vector<hipEvent_t> marks;    // staged path: completion events without timing, likewise
    char *ring[2] = {nullptr, nullptr};   // staged path: page-locked upload and write-back rings
    std::mutex mu;
};

namespace {

constexpr size_t kSlotAlign = 256;

size_t align_up(size_t x) { return (x + kSlotAlign - 1) & ~(kSlotAlign - 1); }

// One array of a layer: host memory, its place in the slot (and in a
// staging buffer laid out like the slot), and the copies it takes part in.
struct Xfer {
    char *host;
    size_t off;
    size_t bytes;
    bool in;     // host -> slot before the step
    bool out;    // slot -> host after the step
};

// A layer's arrays and the launch of its step on a slot.
struct LayerPlan {
    std::vector<Xfer> xfers;
    size_t bytes = 0;                                            // slot bytes used
    std::function<lema_status(char *slot, hipStream_t)> launch;  // step on `slot`
};

struct PlanBuilder {
    LayerPlan *plan;
    // Places an array of `bytes` in the slot; returns its offset.
    size_t add(const void *host, size_t bytes, bool in, bool out) {
        const size_t off = align_up(plan->bytes);
        plan->xfers.push_back({static_cast<char *>(const_cast<void *>(host)), off, bytes, in, out});
        plan->bytes = off + bytes;
        return off;
    }
};

// fp32 state: master, m, v in and out (12 B), bf16 gradient in (2 B), bf16
// weight out (2 B).
LayerPlan plan_fp32(const lema_layer &L, const AdamwConsts &consts) {
    LayerPlan plan;
    PlanBuilder b{&plan};
    struct Offs { size_t master, m, v, grad, weight; int64_t numel; };
    std::vector<Offs> offs;
    for (int32_t i = 0; i < L.nseg; ++i) {
        const lema_adamw_seg &h = L.host_segs[i];
        const size_t n = static_cast<size_t>(h.numel);
        if (n == 0) continue;
        Offs o;
        o.master = b.add(h.master, 4 * n, true, true);
        o.m = b.add(h.exp_avg, 4 * n, true, true);
        o.v = b.add(h.exp_avg_sq, 4 * n, true, true);
        o.grad = b.add(h.grad, 2 * n, true, false);
        o.weight = b.add(h.weight_bf16, 2 * n, false, true);
        o.numel = h.numel;
        offs.push_back(o);
    }
    plan.launch = [offs, consts](char *slot, hipStream_t stream) -> lema_status {
        std::vector<lema_adamw_seg> segs;
        for (const Offs &o : offs) {
            lema_adamw_seg d{};
            d.master = reinterpret_cast<float *>(slot + o.master);
            d.exp_avg = reinterpret_cast<float *>(slot + o.m);
            d.exp_avg_sq = reinterpret_cast<float *>(slot + o.v);
            d.grad = slot + o.grad;
            d.weight_bf16 = reinterpret_cast<uint16_t *>(slot + o.weight);
            d.numel = o.numel;
            segs.push_back(d);
        }
        std::vector<SegRec> recs;
        adamw_records(segs.data(), int32_t(segs.size()), &recs, nullptr);
        return launch_adamw_recs(recs, consts, kGradBf16, stream);
    };
    return plan;
}

// int8 state: master in and out; m and v as codes plus row scales (or fp32)
// in and out; the gradient (bf16, fp32, or int8 codes plus row scales) in;
// the bf16 weight out.
LayerPlan plan_q8(const lema_layer_q8 &L, const lema_adamw_args &args, int32_t moment_dtype) {
    LayerPlan plan;
    PlanBuilder b{&plan};
    const bool mom_q8 = moment_dtype == LEMA_STATE_Q8;
    const bool grad_q8 = args.grad_dtype == LEMA_GRAD_Q8;
    const size_t msize = mom_q8 ? 1 : 4;
    const size_t gsize = args.grad_dtype == LEMA_GRAD_BF16 ? 2 : args.grad_dtype == LEMA_GRAD_FP32 ? 4 : 1;
    struct Offs { size_t master, m, ms, v, vs, grad, gs, weight; int64_t numel, row_len; };
    std::vector<Offs> offs;
    for (int32_t i = 0; i < L.nseg; ++i) {
        const lema_adamw_q8_seg &h = L.host_segs[i];
        const size_t n = static_cast<size_t>(h.numel);
        if (n == 0) continue;
        const size_t rows = (mom_q8 || grad_q8) ? size_t(q8_rows(h.numel, h.row_len)) : 0;
        Offs o{};
        o.master = b.add(h.master, 4 * n, true, true);
        o.m = b.add(h.exp_avg, msize * n, true, true);
        if (mom_q8) o.ms = b.add(h.exp_avg_scale, 4 * rows, true, true);
        o.v = b.add(h.exp_avg_sq, msize * n, true, true);
        if (mom_q8) o.vs = b.add(h.exp_avg_sq_scale, 4 * rows, true, true);
        o.grad = b.add(h.grad, gsize * n, true, false);
        if (grad_q8) o.gs = b.add(h.grad_scale, 4 * rows, true, false);
        o.weight = b.add(h.weight_bf16, 2 * n, false, true);
        o.numel = h.numel;
        o.row_len = h.row_len;
        offs.push_back(o);
    }
    plan.launch = [offs, args, moment_dtype, mom_q8, grad_q8](char *slot,
                                                              hipStream_t stream) -> lema_status {
        std::vector<lema_adamw_q8_seg> segs;
        for (const Offs &o : offs) {
            lema_adamw_q8_seg d{};
            d.master = reinterpret_cast<float *>(slot + o.master);
            d.exp_avg = slot + o.m;
            d.exp_avg_scale = mom_q8 ? reinterpret_cast<float *>(slot + o.ms) : nullptr;
            d.exp_avg_sq = slot + o.v;
            d.exp_avg_sq_scale = mom_q8 ? reinterpret_cast<float *>(slot + o.vs) : nullptr;
            d.grad = slot + o.grad;
            d.grad_scale = grad_q8 ? reinterpret_cast<const float *>(slot + o.gs) : nullptr;
            d.weight_bf16 = reinterpret_cast<uint16_t *>(slot + o.weight);
            d.numel = o.numel;
            d.row_len = o.row_len;
            segs.push_back(d);
        }
        return lema_adamw_step_q8(segs.data(), int32_t(segs.size()), &args, moment_dtype, stream);
    };
    return plan;
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

// Test hook for the failure path: with LEMA_FAULT_INJECT=copy:<n> in the
// environment, the n-th copy (1-based) that one streaming call would enqueue
// is not issued and reports hipErrorUnknown instead.  Nothing reaches the
// GPU; the call then takes its ordinary HIP-failure exit.
struct FaultInjector {
    long fail_at = 0;    // 0: off
    std::atomic<long> count{0};
    FaultInjector() {
        const char *v = std::getenv("LEMA_FAULT_INJECT");
        if (v != nullptr && std::strncmp(v, "copy:", 5) == 0) fail_at = std::atol(v + 5);
    }
    bool fire() { return fail_at > 0 && ++count == fail_at; }
};

hipError_t copy_async(void *dst, const void *src, size_t bytes, hipMemcpyKind kind,
                      hipStream_t s, FaultInjector *fi) {
    if (fi != nullptr && fi->fire()) return hipErrorUnknown;
    return hipMemcpyAsync(dst, src, bytes, kind, s);
}

// Copies of a plan's `in` arrays from the host arrays into the slot.
hipError_t enqueue_upload(const LayerPlan &plan, char *slot, hipStream_t s, double *bytes,
                          FaultInjector *fi) {
    hipError_t e = hipSuccess;
    for (const Xfer &x : plan.xfers) {
        if (!x.in || x.bytes == 0) continue;
        e = copy_async(slot + x.off, x.host, x.bytes, hipMemcpyHostToDevice, s, fi);
        if (e != hipSuccess) return e;
        *bytes += double(x.bytes);
    }
    return e;
}

// Copies of a plan's `out` arrays from the slot back to the host arrays.
hipError_t enqueue_writeback(const LayerPlan &plan, char *slot, hipStream_t s, double *bytes,
                             FaultInjector *fi) {
    hipError_t e = hipSuccess;
    for (const Xfer &x : plan.xfers) {
        if (!x.out || x.bytes == 0) continue;
        e = copy_async(x.host, slot + x.off, x.bytes, hipMemcpyDeviceToHost, s, fi);
        if (e != hipSuccess) return e;
        *bytes += double(x.bytes);
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

// A fixed set of host threads for memcpy.  copy(items) splits the items'
// bytes evenly over the threads, the caller's included, and returns when all
// are copied.  One caller at a time.  If the system refuses a thread, the
// set works with the threads it got (at least the caller's).
class CopyWorkers {
public:
    explicit CopyWorkers(int threads) {
        const int want = std::max(1, threads);
        for (int t = 1; t < want; ++t) {
            try {
                threads_.emplace_back([this, t] { loop(t); });
            } catch (...) {
                break;
            }
        }
        n_ = 1 + int(threads_.size());
    }
    ~CopyWorkers() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
            ++gen_;
        }
        cv_.notify_all();
        for (std::thread &t : threads_) t.join();
    }
    void copy(const CopyItem *items, size_t nitems) {
        size_t total = 0;
        for (size_t i = 0; i < nitems; ++i) total += items[i].bytes;
        if (n_ == 1 || total < (size_t(4) << 20)) {
            for (size_t i = 0; i < nitems; ++i) std::memcpy(items[i].dst, items[i].src, items[i].bytes);
            return;
        }
        {
            std::lock_guard<std::mutex> lk(mu_);
            items_ = items;
            nitems_ = nitems;
            total_ = total;
            share_ = ((total + n_ - 1) / n_ + 63) & ~size_t(63);
            pending_ = n_ - 1;
            ++gen_;
        }
        cv_.notify_all();
        run(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_.wait(lk, [this] { return pending_ == 0; });
    }

private:
    // thread t's share: bytes [t*share, (t+1)*share) of the items laid end to end
    void run(int t) {
        const size_t begin = size_t(t) * share_, end = std::min(total_, begin + share_);
        size_t pos = 0;
        for (size_t i = 0; i < nitems_ && pos < end; ++i) {
            const CopyItem &c = items_[i];
            const size_t lo = std::max(begin, pos), hi = std::min(end, pos + c.bytes);
            if (lo < hi)
                std::memcpy(static_cast<char *>(c.dst) + (lo - pos),
                            static_cast<const char *>(c.src) + (lo - pos), hi - lo);
            pos += c.bytes;
        }
    }
    void loop(int t) {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(mu_);
        for (;;) {
            cv_.wait(lk, [&] { return gen_ != seen; });
            seen = gen_;
            if (stop_) return;
            lk.unlock();
            run(t);
            lk.lock();
            if (--pending_ == 0) done_.notify_one();
        }
    }

    int n_ = 1;
    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable cv_, done_;
    uint64_t gen_ = 0;
    bool stop_ = false;
    const CopyItem *items_ = nullptr;
    size_t nitems_ = 0, total_ = 0, share_ = 0;
    int pending_ = 0;
};

// The staged path moves a layer's arrays in pieces of at most one ring chunk
// through two page-locked rings, one per direction, so that a layer's first
// upload starts after one chunk's host copy and a write-back's host copies
// follow its DMA chunk by chunk.  Back-to-back 128 MiB copies run at the
// rate of one 2 GiB copy on MI355X; a ring of 8 chunks of 128 MiB starved
// the copy engine on the whole 7B shape, 16 kept it busy.
constexpr size_t kStageChunk = size_t(128) << 20;
constexpr int kStageRing = 16;              // chunks per ring (2 GiB)

// One piece of a layer's transfer in one direction: a span of the slot of
// at most one chunk, holding whole or partial arrays that follow each other
// in the slot with only alignment padding between them.  A piece moves as
// one copy between the slot and a ring chunk laid out like the span, and as
// one host copy per part between the chunk and the caller's arrays.  (The
// upload carries the padding's stale ring bytes into slot padding, which no
// array uses.)
struct PiecePart {
    char *host;
    size_t at;        // offset in the span and in the chunk
    size_t bytes;
};
struct Piece {
    size_t slot_off;
    size_t span;
    std::vector<PiecePart> parts;
    size_t bytes() const {
        size_t b = 0;
        for (const PiecePart &q : parts) b += q.bytes;
        return b;
    }
};

void plan_pieces(const LayerPlan &plan, bool inbound, std::vector<Piece> *out) {
    out->clear();
    bool open = false;
    for (const Xfer &x : plan.xfers) {
        if (x.bytes == 0 || (inbound ? !x.in : !x.out)) continue;
        for (size_t done = 0; done < x.bytes;) {
            const size_t off = x.off + done;
            const bool extend = open && off == align_up(out->back().slot_off + out->back().span) &&
                                off - out->back().slot_off < kStageChunk;
            if (!extend) {
                out->push_back({off, 0, {}});
                open = true;
            }
            Piece &p = out->back();
            const size_t at = off - p.slot_off;
            const size_t take = std::min(x.bytes - done, kStageChunk - at);
            p.parts.push_back({x.host + done, at, take});
            p.span = at + take;
            done += take;
        }
    }
}

lema_status validate_layers(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                            const lema_adamw_args *args, std::vector<Span> *spans,
                            std::vector<LayerPlan> *plans) {
    if (pool == nullptr) return LEMA_ERR_NULL;
    lema_status st = check_hparams(args);
    if (st != LEMA_OK) return st;
    if (args->grad_dtype != LEMA_GRAD_BF16) return LEMA_ERR_DTYPE;
    if (nlayers < 0) return LEMA_ERR_SIZE;
    if (nlayers > 0 && layers == nullptr) return LEMA_ERR_NULL;
    const AdamwConsts consts = derive_consts(args);
    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer &L = layers[i];
        st = validate_adamw_segs(L.host_segs, L.nseg, LEMA_GRAD_BF16, false, spans);
        if (st != LEMA_OK) return st;
        plans->push_back(plan_fp32(L, consts));
        if (plans->back().bytes > pool->slot_bytes) return LEMA_ERR_SIZE;
    }
    if (any_conflict(*spans)) return LEMA_ERR_OVERLAP;
    return LEMA_OK;
}

lema_status validate_layers_q8(lema_slot_pool *pool, const lema_layer_q8 *layers,
                               int32_t nlayers, const lema_adamw_args *args,
                               int32_t moment_dtype, std::vector<Span> *spans,
                               std::vector<LayerPlan> *plans) {
    if (pool == nullptr) return LEMA_ERR_NULL;
    lema_status st = check_hparams(args, true);
    if (st != LEMA_OK) return st;
    if (moment_dtype != LEMA_STATE_FP32 && moment_dtype != LEMA_STATE_Q8) return LEMA_ERR_DTYPE;
    if (nlayers < 0) return LEMA_ERR_SIZE;
    if (nlayers > 0 && layers == nullptr) return LEMA_ERR_NULL;
    for (int32_t i = 0; i < nlayers; ++i) {
        const lema_layer_q8 &L = layers[i];
        st = validate_q8_segs(L.host_segs, L.nseg, args->grad_dtype, moment_dtype, false, spans,
                              nullptr, nullptr);
        if (st != LEMA_OK) return st;
        plans->push_back(plan_q8(L, *args, moment_dtype));
        if (plans->back().bytes > pool->slot_bytes) return LEMA_ERR_SIZE;
    }
    if (any_conflict(*spans)) return LEMA_ERR_OVERLAP;
    return LEMA_OK;
}

// Host arrays used straight by the copy engines must be page-locked.
lema_status check_pinned(const std::vector<Span> &spans) {
    for (const Span &s : spans)
        if (s.hi > s.lo && !is_pinned(reinterpret_cast<const void *>(s.lo), s.hi - s.lo))
            return LEMA_ERR_NOT_PINNED;
    return LEMA_OK;
}

// ------------------------------------------------------------- pipelines

// After a failure in the middle of a pipeline: wait for whatever was already
// enqueued on the pool's streams, so that no copy still reads or writes the
// caller's memory once the call has returned.  Returns `st`.
lema_status drain(lema_slot_pool *pool, lema_status st) {
    for (hipStream_t s : {pool->copy, pool->compute, pool->writeback})
        if (s != nullptr) (void)hipStreamSynchronize(s);
    return st;
}

// Page-locked host arrays: copies go straight between host and slots.
lema_status run_direct(lema_slot_pool *pool, const std::vector<LayerPlan> &plans,
                       lema_stream_stats *stats) {
    const int32_t nlayers = int32_t(plans.size());
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
    lema_status st = ensure_events(pool, size_t(nlayers) * EV_PER_LAYER);
    if (st != LEMA_OK) return st;

    auto ev = [&](int layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    auto slot_of = [&](int i) { return pool->base + size_t(i % pool->nslots) * pool->slot_bytes; };
    double h2d_bytes = 0, d2h_bytes = 0;
    FaultInjector fi;
    hipStream_t d2h_stream = pool->writeback ? pool->writeback : pool->copy;

    auto copy_back = [&](int j) -> lema_status {
        hipError_t err = hipStreamWaitEvent(d2h_stream, ev(j, EV_K_END), 0);
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_BEGIN), d2h_stream);
        if (err == hipSuccess) err = enqueue_writeback(plans[j], slot_of(j), d2h_stream, &d2h_bytes, &fi);
        if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_END), d2h_stream);
        return err == hipSuccess ? LEMA_OK : hip_failed(err);
    };

    for (int32_t i = 0; i < nlayers; ++i) {
        // host -> slot; with a separate write-back stream the slot must first
        // have been copied back from its previous occupant
        e = hipSuccess;
        if (pool->writeback && i >= pool->nslots)
            e = hipStreamWaitEvent(pool->copy, ev(i - pool->nslots, EV_D2H_END), 0);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_H2D_BEGIN), pool->copy);
        if (e == hipSuccess) e = enqueue_upload(plans[i], slot_of(i), pool->copy, &h2d_bytes, &fi);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_H2D_END), pool->copy);
        if (e != hipSuccess) return drain(pool, hip_failed(e));

        // the step on the slot
        e = hipStreamWaitEvent(pool->compute, ev(i, EV_H2D_END), 0);
        if (e == hipSuccess) e = hipEventRecord(ev(i, EV_K_BEGIN), pool->compute);
        if (e != hipSuccess) return drain(pool, hip_failed(e));
        st = plans[i].launch(slot_of(i), pool->compute);
        if (st != LEMA_OK) return drain(pool, st);
        e = hipEventRecord(ev(i, EV_K_END), pool->compute);
        if (e != hipSuccess) return drain(pool, hip_failed(e));

        // slot -> host for the previous layer, behind this layer's upload
        if (i >= 1) {
            st = copy_back(i - 1);
            if (st != LEMA_OK) return drain(pool, st);
        }
    }
    st = copy_back(nlayers - 1);
    if (st != LEMA_OK) return drain(pool, st);
    e = hipEventSynchronize(ev(nlayers - 1, EV_D2H_END));
    if (e != hipSuccess) return drain(pool, hip_failed(e));

    if (stats) {
        fill_stats(pool, nlayers, h2d_bytes, d2h_bytes, stats);
        stats->call_ms = std::chrono::duration<double, std::milli>(
                             std::chrono::steady_clock::now() - call_start).count();
    }
    return LEMA_OK;
}

// Pageable or memory-mapped host arrays.  Arrays move in pieces of at most
// one chunk: caller memory -> upload ring -> slot, and slot -> write-
// back ring -> caller memory.  The calling thread copies pieces into the
// upload ring and enqueues their uploads and each layer's step; a second
// thread enqueues the write-backs and copies their pieces out as they land.
//
//   - Completion is tracked per group of kStageGroup pieces: one event
//     without timing after each group.  An event recorded between two copies
//     costs the copy engine about 5 us (MI355X, timing or not), so an event
//     per piece would add milliseconds to a step of ~1,500 pieces.
//   - A ring chunk is reused only after the group of its previous piece is
//     done: uploaded, or written back and copied out.
//   - Layer i's uploads into slot i mod nslots follow the write-back of
//     layer i - nslots out of that slot.
//   - On a single copy stream a layer's write-back is enqueued after the
//     next layer's uploads, so the copy engine never waits for the step in
//     between (the step of layer i runs while layer i+1 uploads).
//   - Timing events are per layer and direction, as in run_direct: the copy
//     intervals run from the first piece's start to the last piece's end.
constexpr int kStageGroup = 4;

lema_status ensure_marks(lema_slot_pool *pool, size_t n) {
    while (pool->marks.size() < n) {
        hipEvent_t ev;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_failed(e);
        pool->marks.push_back(ev);
    }
    return LEMA_OK;
}

// groups of a transfer of n pieces that end before its last piece
size_t inner_groups(size_t n) { return n == 0 ? 0 : (n - 1) / kStageGroup; }

lema_status run_staged(lema_slot_pool *pool, const std::vector<LayerPlan> &plans,
                       int32_t host_threads, lema_stream_stats *stats) {
    const int32_t nlayers = int32_t(plans.size());
    if (nlayers == 0) {
        if (stats) *stats = lema_stream_stats{};
        return LEMA_OK;
    }
    int threads = host_threads;
    if (threads == 0) {
        const unsigned hc = std::thread::hardware_concurrency();
        threads = int(std::min(16u, hc == 0 ? 4u : hc));
    }
    const int threads_in = std::max(1, threads / 2), threads_out = std::max(1, threads - threads_in);
    using clock = std::chrono::steady_clock;
    const auto call_start = clock::now();

    std::lock_guard<std::mutex> lock(pool->mu);
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_failed(e);
    if (cur != pool->device) return LEMA_ERR_HIP;
    for (char *&r : pool->ring) {
        if (r == nullptr) {
            e = hipHostMalloc(reinterpret_cast<void **>(&r), kStageChunk * kStageRing,
                              hipHostMallocDefault);
            if (e != hipSuccess) {
                r = nullptr;
                return hip_failed(e);
            }
        }
    }
    std::vector<std::vector<Piece>> in_p(nlayers), out_p(nlayers);
    std::vector<size_t> in_mark(nlayers), out_mark(nlayers);   // first inner-group mark per layer
    size_t n_in = 0, n_out = 0, n_marks = 0;
    for (int32_t i = 0; i < nlayers; ++i) {
        plan_pieces(plans[i], true, &in_p[i]);
        plan_pieces(plans[i], false, &out_p[i]);
        n_in += in_p[i].size();
        n_out += out_p[i].size();
        in_mark[i] = n_marks;
        n_marks += inner_groups(in_p[i].size());
        out_mark[i] = n_marks;
        n_marks += inner_groups(out_p[i].size());
    }
    if (n_in == 0 || n_out == 0) {                 // only empty segments: nothing moves
        if (stats) *stats = lema_stream_stats{};
        return LEMA_OK;
    }
    lema_status st = ensure_events(pool, size_t(nlayers) * EV_PER_LAYER);
    if (st == LEMA_OK) st = ensure_marks(pool, n_marks);
    if (st != LEMA_OK) return st;
    auto ev = [&](int32_t layer, int kind) { return pool->events[size_t(layer) * EV_PER_LAYER + kind]; };
    auto slot_of = [&](int32_t i) { return pool->base + size_t(i % pool->nslots) * pool->slot_bytes; };
    // The event that completes piece k of a transfer of n pieces: the mark
    // of its group, or for the last group the transfer's own end event.
    auto group_event = [&](size_t first_mark, size_t k, size_t n, hipEvent_t end) {
        const size_t g = k / kStageGroup;
        return g < inner_groups(n) ? pool->marks[first_mark + g] : end;
    };
    auto closes_group = [](size_t k, size_t n) { return k + 1 == n || (k + 1) % kStageGroup == 0; };

    const bool duplex = pool->writeback != nullptr;
    hipStream_t d2h_stream = duplex ? pool->writeback : pool->copy;
    FaultInjector fi;

    // progress shared by the two threads
    std::mutex m;
    std::condition_variable cv;
    int32_t steps_enqueued = 0;     // layers whose uploads and step are enqueued
    int32_t backs_enqueued = 0;     // layers whose write-backs are enqueued
    bool abort = false;
    lema_status out_status = LEMA_OK;
    int32_t out_hip = 0;            // the write-back thread's HIP error, if it failed
    double h2d_bytes = 0, d2h_bytes = 0, in_ms = 0, out_ms = 0;

    auto fail = [&](lema_status s2) {
        std::lock_guard<std::mutex> lk(m);
        abort = true;
        return s2;
    };

    auto outbound_work = [&] {
        // HIP's current device is per thread: this one starts on device 0
        lema_status s2 = LEMA_OK;
        hipError_t err = hipSetDevice(pool->device);
        if (err != hipSuccess) s2 = hip_failed(err);
        CopyWorkers workers(threads_out);
        struct Pending { hipEvent_t done; char *chunk; const Piece *piece; };
        std::deque<Pending> fifo;          // enqueued pieces not yet copied out, oldest first
        std::vector<CopyItem> batch;
        size_t next = 0;
        // copy out the oldest group: every pending piece that its event completes
        auto complete_oldest = [&]() -> lema_status {
            const hipEvent_t done = fifo.front().done;
            hipError_t err = hipEventSynchronize(done);
            if (err != hipSuccess) return hip_failed(err);
            batch.clear();
            while (!fifo.empty() && fifo.front().done == done) {
                for (const PiecePart &q : fifo.front().piece->parts)
                    batch.push_back({q.host, fifo.front().chunk + q.at, q.bytes});
                fifo.pop_front();
            }
            const auto t0 = clock::now();
            workers.copy(batch.data(), batch.size());
            out_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
            return LEMA_OK;
        };
        for (int32_t j = 0; j < nlayers && s2 == LEMA_OK; ++j) {
            {
                // the step of layer j enqueued, and on a single copy stream also
                // the uploads of layer j + 1
                std::unique_lock<std::mutex> lk(m);
                const int32_t need = (duplex || j == nlayers - 1) ? j + 1 : j + 2;
                cv.wait(lk, [&] { return abort || steps_enqueued >= need; });
                if (abort) break;
            }
            err = hipStreamWaitEvent(d2h_stream, ev(j, EV_K_END), 0);
            if (err == hipSuccess) err = hipEventRecord(ev(j, EV_D2H_BEGIN), d2h_stream);
            if (err != hipSuccess) { s2 = hip_failed(err); break; }
            char *slot = slot_of(j);
            const size_t n = out_p[j].size();
            for (size_t k = 0; k < n; ++k) {
                if (fifo.size() == size_t(kStageRing)) {
                    s2 = complete_oldest();
                    if (s2 != LEMA_OK) break;
                }
                const Piece &p = out_p[j][k];
                char *chunk = pool->ring[1] + (next++ % kStageRing) * kStageChunk;
                err = copy_async(chunk, slot + p.slot_off, p.span, hipMemcpyDeviceToHost,
                                 d2h_stream, &fi);
                const hipEvent_t done = group_event(out_mark[j], k, n, ev(j, EV_D2H_END));
                if (err == hipSuccess && closes_group(k, n)) err = hipEventRecord(done, d2h_stream);
                if (err != hipSuccess) { s2 = hip_failed(err); break; }
                d2h_bytes += double(p.bytes());
                fifo.push_back({done, chunk, &p});
            }
            if (s2 != LEMA_OK) break;
            if (n == 0) {
                err = hipEventRecord(ev(j, EV_D2H_END), d2h_stream);
                if (err != hipSuccess) { s2 = hip_failed(err); break; }
            }
            {
                std::lock_guard<std::mutex> lk(m);
                backs_enqueued = j + 1;
            }
            cv.notify_all();
        }
        while (s2 == LEMA_OK && !fifo.empty()) {
            bool stop;
            {
                std::lock_guard<std::mutex> lk(m);
                stop = abort;
            }
            if (stop) break;
            s2 = complete_oldest();
        }
        if (s2 != LEMA_OK) {
            std::lock_guard<std::mutex> lk(m);
            abort = true;
            out_status = s2;
            out_hip = lema_last_hip_error();   // this thread's; handed to the caller's below
        }
        cv.notify_all();
    };
    std::thread outbound;
    try {
        outbound = std::thread(outbound_work);
    } catch (...) {                        // nothing is enqueued yet
        return hip_failed(hipErrorOutOfMemory);
    }

    // this thread: uploads and steps
    st = LEMA_OK;
    {
        CopyWorkers workers(threads_in);
        std::vector<hipEvent_t> chunk_done(kStageRing, nullptr);   // completes a chunk's last upload
        std::vector<size_t> open;                                  // chunks of the group being enqueued
        std::vector<CopyItem> items;
        size_t next = 0;
        for (int32_t i = 0; i < nlayers && st == LEMA_OK; ++i) {
            {
                std::lock_guard<std::mutex> lk(m);
                if (abort) break;
            }
            if (i >= pool->nslots) {
                // the slot's previous occupant is written back first: on one
                // copy stream by the order of enqueueing, else by its event
                std::unique_lock<std::mutex> lk(m);
                cv.wait(lk, [&] { return abort || backs_enqueued >= i - pool->nslots + 1; });
                if (abort) break;
                lk.unlock();
                if (duplex) {
                    e = hipStreamWaitEvent(pool->copy, ev(i - pool->nslots, EV_D2H_END), 0);
                    if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
                }
            }
            e = hipEventRecord(ev(i, EV_H2D_BEGIN), pool->copy);
            if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
            char *slot = slot_of(i);
            const size_t n = in_p[i].size();
            for (size_t k = 0; k < n; ++k) {
                const Piece &p = in_p[i][k];
                const size_t c = next++ % kStageRing;
                if (chunk_done[c] != nullptr) {
                    e = hipEventSynchronize(chunk_done[c]);
                    if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
                }
                char *chunk = pool->ring[0] + c * kStageChunk;
                items.clear();
                for (const PiecePart &q : p.parts) items.push_back({chunk + q.at, q.host, q.bytes});
                const auto t0 = clock::now();
                workers.copy(items.data(), items.size());
                in_ms += std::chrono::duration<double, std::milli>(clock::now() - t0).count();
                e = copy_async(slot + p.slot_off, chunk, p.span, hipMemcpyHostToDevice,
                               pool->copy, &fi);
                if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
                h2d_bytes += double(p.bytes());
                open.push_back(c);
                if (closes_group(k, n)) {
                    const hipEvent_t done = group_event(in_mark[i], k, n, ev(i, EV_H2D_END));
                    e = hipEventRecord(done, pool->copy);
                    if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
                    for (size_t oc : open) chunk_done[oc] = done;
                    open.clear();
                }
            }
            if (st != LEMA_OK) break;
            if (n == 0) {
                e = hipEventRecord(ev(i, EV_H2D_END), pool->copy);
                if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
            }
            e = hipStreamWaitEvent(pool->compute, ev(i, EV_H2D_END), 0);
            if (e == hipSuccess) e = hipEventRecord(ev(i, EV_K_BEGIN), pool->compute);
            if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
            st = plans[i].launch(slot, pool->compute);
            if (st != LEMA_OK) { fail(st); break; }
            e = hipEventRecord(ev(i, EV_K_END), pool->compute);
            if (e != hipSuccess) { st = fail(hip_failed(e)); break; }
            {
                std::lock_guard<std::mutex> lk(m);
                steps_enqueued = i + 1;
            }
            cv.notify_all();
        }
        cv.notify_all();
    }
    outbound.join();
    if (st == LEMA_OK && out_status != LEMA_OK) {
        st = out_status;
        if (st == LEMA_ERR_HIP) hip_failed(static_cast<hipError_t>(out_hip));
    }
    if (st != LEMA_OK) return drain(pool, st);
    e = hipEventSynchronize(ev(nlayers - 1, EV_D2H_END));
    if (e != hipSuccess) return drain(pool, hip_failed(e));

    if (stats) {
        fill_stats(pool, nlayers, h2d_bytes, d2h_bytes, stats);
        stats->host_in_ms = in_ms;
        stats->host_out_ms = out_ms;
        stats->call_ms = std::chrono::duration<double, std::milli>(clock::now() - call_start).count();
    }
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
        for (hipEvent_t ev : pool->marks) {
            hipError_t e = hipEventSynchronize(ev);
            if (e != hipSuccess && e != hipErrorInvalidResourceHandle && st == LEMA_OK) st = hip_failed(e);
            (void)hipEventDestroy(ev);
        }
        pool->marks.clear();
        for (char *&p : pool->ring) {
            if (p) (void)hipHostFree(p);
            p = nullptr;
        }
    }
    delete pool;
    return st;
}

lema_status lema_slot_stream(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                             const lema_adamw_args *args, lema_stream_stats *stats) {
    // validation of every layer before anything is enqueued
    std::vector<Span> spans;
    std::vector<LayerPlan> plans;
    lema_status st = validate_layers(pool, layers, nlayers, args, &spans, &plans);
    if (st != LEMA_OK) return st;
    st = check_pinned(spans);
    if (st != LEMA_OK) return st;
    return run_direct(pool, plans, stats);
}

lema_status lema_slot_stream_staged(lema_slot_pool *pool, const lema_layer *layers,
                                    int32_t nlayers, const lema_adamw_args *args,
                                    int32_t host_threads, lema_stream_stats *stats) {
    std::vector<Span> spans;
    std::vector<LayerPlan> plans;
    lema_status st = validate_layers(pool, layers, nlayers, args, &spans, &plans);
    if (st != LEMA_OK) return st;
    if (host_threads < 0 || host_threads > 256) return LEMA_ERR_SIZE;
    return run_staged(pool, plans, host_threads, stats);
}

lema_status lema_slot_stream_q8(lema_slot_pool *pool, const lema_layer_q8 *layers,
                                int32_t nlayers, const lema_adamw_args *args,
                                int32_t moment_dtype, int32_t staged, int32_t host_threads,
                                lema_stream_stats *stats) {
    std::vector<Span> spans;
    std::vector<LayerPlan> plans;
    lema_status st = validate_layers_q8(pool, layers, nlayers, args, moment_dtype, &spans, &plans);
    if (st != LEMA_OK) return st;
    if (staged) {
        if (host_threads < 0 || host_threads > 256) return LEMA_ERR_SIZE;
        return run_staged(pool, plans, host_threads, stats);
    }
    st = check_pinned(spans);
    if (st != LEMA_OK) return st;
    return run_direct(pool, plans, stats);
}

}  // extern "C"
