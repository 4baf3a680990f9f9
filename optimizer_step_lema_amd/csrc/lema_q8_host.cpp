// lema_q8_host.cpp -- host side of the int8 + per-row-scale entry points of
// include/lema.h: validation, row-team sizing, launch tables and launches.
//
// Method: LEMA README, "Quantization" (8-bit optimizer state and gradient
// accumulators: int8 codes with a scale per row, widened to fp32 within the
// step).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "lema.h"
#include "lema_measure.h"
#include "lema_host_internal.h"
#include "lema_internal.h"

namespace lema {
namespace {

static_assert(kQMaxRow == LEMA_Q8_MAX_ROW, "row limit of the header and the kernels agree");
static_assert(int64_t(kQBlock) * kQWaveCodeChunks * 4 >= kQMaxRow,
              "wave-row accumulation and conversions need only kQBlock-lane workgroups");

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Team width (log2), chunks per lane and workgroup size for rows of row_len
// elements: the narrowest team whose lanes hold at most `chunks_max` chunks
// in a kQBlock-lane workgroup, else a team of a kQBlockWide-lane workgroup
// with at most kQWideChunks per lane.  Wave rows use teams of at least one
// wavefront (min_log2w = 6).
struct Shape {
    int32_t log2w, chunks;
    int block;
};

Shape shape_for(int64_t row_len, int chunks_max, int min_log2w = 0) {
    const int64_t need = ceil_div(row_len, 4);
    int lg = min_log2w;
    while ((1 << lg) < kQBlock && ceil_div(need, int64_t(1) << lg) > chunks_max) ++lg;
    if (ceil_div(need, int64_t(1) << lg) <= chunks_max)
        return {lg, static_cast<int32_t>(ceil_div(need, int64_t(1) << lg)), kQBlock};
    lg = min_log2w;
    while (ceil_div(need, int64_t(1) << lg) > kQWideChunks) ++lg;
    return {lg, static_cast<int32_t>(ceil_div(need, int64_t(1) << lg)), kQBlockWide};
}

// Rows of 4*S elements, S a power of two up to 64 lanes, go packed: a team
// of S lanes covers the row in one chunk step and each lane's chunks hold
// `chunks_max` different rows (contiguous accesses across the wavefront).
bool packed_row_len(int64_t row_len) {
    if (row_len < 4 || row_len > 256 || row_len % 4 != 0) return false;
    const int64_t s = row_len / 4;
    return (s & (s - 1)) == 0;
}

uint64_t blocks_of(const Q8Rec &r) {
    int64_t rows_per_block = r.block >> r.team_log2;
    if (r.flags & kQPacked) rows_per_block *= r.chunks;
    return static_cast<uint64_t>(ceil_div(r.rows, rows_per_block));
}

bool row_len_ok(int64_t row_len) { return row_len >= 1 && row_len <= kQMaxRow; }

// The record of one segment.  Vector-aligned rows go packed (4 .. 256
// elements, S a power of two), or as wave rows when the segment's element
// count is a multiple of 4 and a row spans at least 64 vectors (teams of
// whole wavefronts holding up to `wave_chunks` chunks per lane); everything
// else goes to row teams of at most `chunks_max` chunks per lane.
Q8Rec make_rec(int64_t numel, int64_t row_len, bool vector_ok, int chunks_max, int wave_chunks) {
    Q8Rec r{};
    r.numel = numel;
    r.row_len = row_len;
    r.rows = ceil_div(numel, row_len);
    const Shape sh = shape_for(row_len, chunks_max);
    r.team_log2 = sh.log2w;
    r.chunks = sh.chunks;
    r.block = sh.block;
    r.flags = (vector_ok && row_len % 4 == 0) ? kQVector : 0;
    if (r.flags && packed_row_len(row_len)) {
        int lg = 0;
        while ((int64_t(4) << lg) < row_len) ++lg;
        r.team_log2 = lg;
        r.chunks = chunks_max;
        r.block = kQBlock;
        r.flags |= kQPacked;
    } else if (r.flags && row_len >= 256 && numel % 4 == 0) {
        const Shape w = shape_for(row_len, wave_chunks, 6);
        r.team_log2 = w.log2w;
        r.chunks = w.chunks;
        r.block = w.block;
        r.flags |= kQWave;
    }
    return r;
}

QRows rows_of(const Q8Rec &r) {
    if (r.flags & kQMixed) return kQRowsMixed;
    return (r.flags & kQPacked) ? kQRowsPacked : (r.flags & kQWave) ? kQRowsWave : kQRowsTeam;
}

// The step's packed-row and wave-row records go into one mixed launch when
// they would otherwise take more than one launch group, every such group is
// small enough that its ramp and drain weigh (at most kMixRounds rounds of
// workgroups over the GPU at the step's occupancy), and every wave row fits
// a kQBlock-lane team of at most kQMixedWaveChunks chunks per lane (rows of
// up to 11,264 elements).  Measured on MI355X: the rank-16 LoRA step (three
// groups of 0.7 to 21 rounds) ran 4-5% faster in one launch, while the
// whole 7B shape (groups of hundreds of rounds) ran 4-9% slower, and one
// Llama-2-7B layer (40 rounds) the same.  Rows that the separate launches
// give 1024-lane workgroups get one 256-lane team each; the others keep
// their shape.  The records are ordered by the work of one of their
// workgroups, the largest first, so that the long rows start early and the
// short ones fill the end of the launch.
constexpr int64_t kMixRounds = 16;

void mix_step_records(std::vector<Q8Rec> *recs, int cus) {
    uint64_t packed = 0, wave = 0, wide = 0;    // workgroups of each separate group
    for (const Q8Rec &r : *recs) {
        if (r.flags & kQPacked) {
            packed += blocks_of(r);
        } else if (r.flags & kQWave) {
            if (r.block == kQBlock) {
                wave += blocks_of(r);
            } else {
                wide += blocks_of(r);
                if (ceil_div(r.row_len, 4) > int64_t(kQBlock) * kQMixedWaveChunks) return;
            }
        }
    }
    if (int(packed > 0) + int(wave > 0) + int(wide > 0) < 2) return;
    const uint64_t round = uint64_t(std::max(cus, 1)) * kQ8StepWorkgroupsPerCu;
    if (std::max({packed, wave, wide}) > uint64_t(kMixRounds) * round) return;
    for (Q8Rec &r : *recs) {
        if (!(r.flags & (kQPacked | kQWave))) continue;
        if ((r.flags & kQWave) && r.block != kQBlock) {
            r.team_log2 = 8;                                  // kQBlock lanes
            r.chunks = static_cast<int32_t>(ceil_div(ceil_div(r.row_len, 4), kQBlock));
            r.block = kQBlock;
        }
        r.flags |= kQMixed;
    }
    // every lane of a kQBlock-lane workgroup steps 4 elements per chunk, so
    // a workgroup's work is its record's chunk count
    auto work = [](const Q8Rec &r) { return (r.flags & kQMixed) ? r.chunks : 0; };
    std::stable_sort(recs->begin(), recs->end(),
                     [&](const Q8Rec &a, const Q8Rec &b) { return work(a) > work(b); });
}

uintptr_t bits(const void *p) { return reinterpret_cast<uintptr_t>(p); }

// Launch `recs` in at most six groups, one per kernel: the step's mixed
// records, row teams and wave rows in kQBlock- or kQBlockWide-lane
// workgroups, and packed rows.  Every
// group's table is built and checked before the first launch, so a size
// error enqueues nothing.
template <class LaunchFn>
lema_status launch_groups(const std::vector<Q8Rec> &recs, hipStream_t stream,
                          const LaunchFn &launch) {
    struct Group {
        int block;
        QRows rows;
        int n;
        uint64_t blocks;
        std::vector<unsigned char> bytes;
    };
    std::vector<Group> groups;
    const struct { int block; QRows rows; } kinds[] = {
        {kQBlock, kQRowsMixed}, {kQBlock, kQRowsTeam}, {kQBlock, kQRowsPacked},
        {kQBlock, kQRowsWave}, {kQBlockWide, kQRowsTeam}, {kQBlockWide, kQRowsWave}};
    for (const auto &kind : kinds) {
        std::vector<Q8Rec> sel;
        for (const Q8Rec &r : recs)
            if (r.block == kind.block && rows_of(r) == kind.rows) sel.push_back(r);
        if (sel.empty()) continue;
        Group g{kind.block, kind.rows, static_cast<int>(sel.size()), 0, {}};
        g.bytes.assign(q8_table_bytes(g.n), 0);
        uint32_t *begin = reinterpret_cast<uint32_t *>(g.bytes.data());
        for (int i = 0; i < g.n; ++i) {
            begin[i] = static_cast<uint32_t>(g.blocks);
            g.blocks += blocks_of(sel[i]);
            if (g.blocks > 0xFFF00000ull) return LEMA_ERR_SIZE;
        }
        begin[g.n] = static_cast<uint32_t>(g.blocks);
        std::memcpy(g.bytes.data() + table_tiles_bytes(g.n), sel.data(), sizeof(Q8Rec) * g.n);
        groups.push_back(std::move(g));
    }
    for (const Group &g : groups) {
        lema_status st = launch_on_table(g.bytes, stream, [&](const void *table) {
            return launch(table, g.n, static_cast<uint32_t>(g.blocks), g.block, g.rows);
        });
        if (st != LEMA_OK) return st;
    }
    return LEMA_OK;
}

// The fp32-moment step with a bf16 or fp32 gradient is the plain step.
lema_status plain_step(const lema_adamw_q8_seg *segs, int32_t nseg, const lema_adamw_args *args,
                       void *stream) {
    std::vector<lema_adamw_seg> plain(static_cast<size_t>(nseg));
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_q8_seg &s = segs[i];
        plain[i] = lema_adamw_seg{s.master, static_cast<float *>(s.exp_avg),
                                  static_cast<float *>(s.exp_avg_sq), s.grad, s.weight_bf16,
                                  s.orig_bf16, s.delta, s.numel};
    }
    return lema_adamw_step(plain.data(), nseg, args, stream);
}

}  // namespace

int64_t q8_rows(int64_t numel, int64_t row_len) { return ceil_div(numel, row_len); }

lema_status validate_q8_segs(const lema_adamw_q8_seg *segs, int32_t nseg, int32_t gd,
                             int32_t moment_dtype, bool delta_allowed, std::vector<Span> *spans,
                             std::vector<Q8Rec> *recs, bool *with_delta) {
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    const bool mom_q8 = moment_dtype == LEMA_STATE_Q8;
    const bool rows_used = mom_q8 || gd == LEMA_GRAD_Q8;
    const size_t mom_size = mom_q8 ? 1 : 4;
    const size_t grad_size = gd == LEMA_GRAD_BF16 ? 2 : gd == LEMA_GRAD_FP32 ? 4 : 1;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_adamw_q8_seg &s = segs[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if ((s.orig_bf16 == nullptr) != (s.delta == nullptr)) return LEMA_ERR_NULL;
        if (!delta_allowed && s.delta != nullptr) return LEMA_ERR_NULL;
        if (s.numel == 0) continue;
        if (rows_used && !row_len_ok(s.row_len)) return LEMA_ERR_SIZE;
        if (!s.master || !s.exp_avg || !s.exp_avg_sq || !s.grad || !s.weight_bf16)
            return LEMA_ERR_NULL;
        if (mom_q8 && (!s.exp_avg_scale || !s.exp_avg_sq_scale)) return LEMA_ERR_NULL;
        if (gd == LEMA_GRAD_Q8 && !s.grad_scale) return LEMA_ERR_NULL;

        // required alignment: each array to its element size
        uintptr_t f32 = bits(s.master) | bits(s.delta) |
                        (mom_q8 ? bits(s.exp_avg_scale) | bits(s.exp_avg_sq_scale)
                                : bits(s.exp_avg) | bits(s.exp_avg_sq)) |
                        (gd == LEMA_GRAD_FP32 ? bits(s.grad) : 0) |
                        (gd == LEMA_GRAD_Q8 ? bits(s.grad_scale) : 0);
        uintptr_t b16 = bits(s.weight_bf16) | bits(s.orig_bf16) |
                        (gd == LEMA_GRAD_BF16 ? bits(s.grad) : 0);
        if ((f32 & 3) || (b16 & 1)) return LEMA_ERR_ALIGN;
        // vector path: 16-byte fp32 arrays, 8-byte bf16, 4-byte codes
        const uintptr_t v16 = bits(s.master) | bits(s.delta) |
                              (mom_q8 ? 0 : bits(s.exp_avg) | bits(s.exp_avg_sq)) |
                              (gd == LEMA_GRAD_FP32 ? bits(s.grad) : 0);
        const uintptr_t v4 = (mom_q8 ? bits(s.exp_avg) | bits(s.exp_avg_sq) : 0) |
                             (gd == LEMA_GRAD_Q8 ? bits(s.grad) : 0);
        const bool vec = (v16 & 15) == 0 && (b16 & 7) == 0 && (v4 & 3) == 0;

        const int64_t rows = rows_used ? q8_rows(s.numel, s.row_len) : 0;
        if (spans) {
            add_span(*spans, s.master, s.numel, 4, true);
            add_span(*spans, s.exp_avg, s.numel, mom_size, true);
            add_span(*spans, s.exp_avg_sq, s.numel, mom_size, true);
            if (mom_q8) {
                add_span(*spans, s.exp_avg_scale, rows, 4, true);
                add_span(*spans, s.exp_avg_sq_scale, rows, 4, true);
            }
            add_span(*spans, s.grad, s.numel, grad_size, false);
            if (gd == LEMA_GRAD_Q8) add_span(*spans, s.grad_scale, rows, 4, false);
            add_span(*spans, s.weight_bf16, s.numel, 2, true);
            if (s.delta) {
                add_span(*spans, s.orig_bf16, s.numel, 2, false);
                add_span(*spans, s.delta, s.numel, 4, true);
            }
        }
        if (s.delta && with_delta) *with_delta = true;
        if (recs) {
            Q8Rec r = make_rec(s.numel, s.row_len, vec, kQStepChunks, kQStepChunks);
            const void *ptrs[10] = {s.master, s.exp_avg, mom_q8 ? s.exp_avg_scale : nullptr,
                                    s.exp_avg_sq, mom_q8 ? s.exp_avg_sq_scale : nullptr, s.grad,
                                    gd == LEMA_GRAD_Q8 ? s.grad_scale : nullptr, s.weight_bf16,
                                    s.orig_bf16, s.delta};
            for (int k = 0; k < 10; ++k) r.p[k] = reinterpret_cast<uint64_t>(ptrs[k]);
            recs->push_back(r);
        }
    }
    return LEMA_OK;
}

}  // namespace lema

using namespace lema;

extern "C" {

lema_status lema_adamw_step_q8(const lema_adamw_q8_seg *segs, int32_t nseg,
                               const lema_adamw_args *args, int32_t moment_dtype, void *stream) {
    lema_status st = check_hparams(args, true);
    if (st != LEMA_OK) return st;
    if (moment_dtype != LEMA_STATE_FP32 && moment_dtype != LEMA_STATE_Q8) return LEMA_ERR_DTYPE;
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    const bool mom_q8 = moment_dtype == LEMA_STATE_Q8;
    const int32_t gd = args->grad_dtype;
    if (!mom_q8 && gd != LEMA_GRAD_Q8) return plain_step(segs, nseg, args, stream);

    std::vector<Span> spans;
    std::vector<Q8Rec> recs;
    bool with_delta = false;
    st = validate_q8_segs(segs, nseg, gd, moment_dtype, true, &spans, &recs, &with_delta);
    if (st != LEMA_OK) return st;
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    if (recs.empty()) return LEMA_OK;
    const AdamwConsts c = derive_consts(args);
    const QGrad qg = gd == LEMA_GRAD_BF16 ? kQGradBf16 : gd == LEMA_GRAD_FP32 ? kQGradF32 : kQGradQ8;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // 256-lane workgroups of the step each stream ~90 KB of state for their
    // row; beyond 3 of them per CU (7 fit by registers) HBM delivers less
    // (measured on MI355X: 2-3% faster at 3 per CU than uncapped on the
    // attention and layer workloads, 1-2% faster than at 4 or 5; 2 per CU
    // starves small launches such as the LoRA adapters).  The 1024-lane
    // ones fit once per CU anyway.  Accumulation and conversions move less
    // per workgroup and keep full occupancy.
    // one mixed launch where its kernel's registers still allow the step's
    // workgroups per CU (some gradient and moment combinations need more)
    if (register_occupancy(adamw_q8_kernel_fn(mom_q8, qg, with_delta, kQBlock, kQRowsMixed),
                           kQBlock) >= kQ8StepWorkgroupsPerCu)
        mix_step_records(&recs, compute_units());
    // (the reservations are looked up here: the launch callback below runs
    // with the device's table cache locked)
    uint32_t lds[4];
    for (QRows rows : {kQRowsTeam, kQRowsPacked, kQRowsWave, kQRowsMixed})
        lds[rows] = occupancy_lds_bytes(adamw_q8_kernel_fn(mom_q8, qg, with_delta, kQBlock, rows),
                                        kQ8StepWorkgroupsPerCu);
    return launch_groups(recs, hs, [&](const void *table, int n, uint32_t blocks,
                                                     int block, QRows rows) {
        return launch_adamw_q8(table, n, blocks, mom_q8, qg, with_delta, block, rows, c, hs,
                               block == kQBlock ? lds[rows] : 0);
    });
}

lema_status lema_grad_accum_q8(const lema_accum_q8_seg *segs, int32_t nseg, int32_t overwrite,
                               void *stream) {
    if (nseg < 0) return LEMA_ERR_SIZE;
    if (nseg > 0 && segs == nullptr) return LEMA_ERR_NULL;
    std::vector<Span> spans;
    std::vector<Q8Rec> recs;
    for (int32_t i = 0; i < nseg; ++i) {
        const lema_accum_q8_seg &s = segs[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if (s.numel == 0) continue;
        if (!row_len_ok(s.row_len)) return LEMA_ERR_SIZE;
        if (!s.acc || !s.acc_scale || !s.grad_bf16) return LEMA_ERR_NULL;
        if ((bits(s.acc_scale) & 3) || (bits(s.grad_bf16) & 1)) return LEMA_ERR_ALIGN;
        const bool vec = (bits(s.acc) & 3) == 0 && (bits(s.grad_bf16) & 7) == 0;
        Q8Rec r = make_rec(s.numel, s.row_len, vec, kQCodeChunks, kQWaveCodeChunks);
        add_span(spans, s.acc, s.numel, 1, true);
        add_span(spans, s.acc_scale, r.rows, 4, true);
        add_span(spans, s.grad_bf16, s.numel, 2, false);
        r.p[0] = reinterpret_cast<uint64_t>(s.acc);
        r.p[1] = reinterpret_cast<uint64_t>(s.acc_scale);
        r.p[2] = reinterpret_cast<uint64_t>(s.grad_bf16);
        recs.push_back(r);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    if (recs.empty()) return LEMA_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return launch_groups(recs, hs, [&](const void *table, int n, uint32_t blocks,
                                                     int block, QRows rows) {
        return launch_accum_q8(table, n, blocks, overwrite != 0, block, rows, hs);
    });
}

static lema_status convert_rows(const lema_q8_tensor *t, int32_t n, bool dequantize,
                                void *stream) {
    if (n < 0) return LEMA_ERR_SIZE;
    if (n > 0 && t == nullptr) return LEMA_ERR_NULL;
    std::vector<Span> spans;
    std::vector<Q8Rec> recs;
    for (int32_t i = 0; i < n; ++i) {
        const lema_q8_tensor &s = t[i];
        if (s.numel < 0) return LEMA_ERR_SIZE;
        if (s.numel == 0) continue;
        if (!row_len_ok(s.row_len)) return LEMA_ERR_SIZE;
        if (!s.x || !s.codes || !s.scale) return LEMA_ERR_NULL;
        if ((bits(s.x) | bits(s.scale)) & 3) return LEMA_ERR_ALIGN;
        const bool vec = (bits(s.x) & 15) == 0 && (bits(s.codes) & 3) == 0;
        Q8Rec r = make_rec(s.numel, s.row_len, vec, kQCodeChunks, kQWaveCodeChunks);
        add_span(spans, s.x, s.numel, 4, dequantize);
        add_span(spans, s.codes, s.numel, 1, !dequantize);
        add_span(spans, s.scale, r.rows, 4, !dequantize);
        r.p[0] = reinterpret_cast<uint64_t>(s.x);
        r.p[1] = reinterpret_cast<uint64_t>(s.codes);
        r.p[2] = reinterpret_cast<uint64_t>(s.scale);
        recs.push_back(r);
    }
    if (any_conflict(spans)) return LEMA_ERR_OVERLAP;
    if (recs.empty()) return LEMA_OK;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return launch_groups(recs, hs, [&](const void *table, int nrec,
                                                     uint32_t blocks, int block, QRows rows) {
        return launch_quantize_q8(table, nrec, blocks, dequantize, block, rows, hs);
    });
}

lema_status lema_probe_q8_reciprocal(const float *s, float *r, int64_t n, void *stream) {
    if (n < 0) return LEMA_ERR_SIZE;
    if (n == 0) return LEMA_OK;
    if (s == nullptr || r == nullptr) return LEMA_ERR_NULL;
    if ((bits(s) | bits(r)) & 3) return LEMA_ERR_ALIGN;
    const hipError_t e = launch_q8_recip_probe(s, r, n, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LEMA_OK : hip_failed(e);
}

lema_status lema_quantize_rows(const lema_q8_tensor *t, int32_t n, void *stream) {
    return convert_rows(t, n, false, stream);
}

lema_status lema_dequantize_rows(const lema_q8_tensor *t, int32_t n, void *stream) {
    return convert_rows(t, n, true, stream);
}

}  // extern "C"
