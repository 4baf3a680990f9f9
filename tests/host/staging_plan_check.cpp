// Host-only check of the staged path's piece planner (plan_pieces in
// lema_slot.cpp), built by tests/test_staging_plan.py.  Random slot layouts
// of arrays in either or both directions, sizes from a few bytes to several
// ring chunks; for each direction it checks that
//   - every piece spans at most one ring chunk and starts 256-byte aligned;
//   - a piece's parts lie in order inside its span, the span ends with its
//     last part, and no array of the other direction overlaps the span
//     (the upload writes a piece's whole span into the slot);
//   - each part maps to the right host bytes of an array of that direction;
//   - the parts cover every byte of every array of that direction once.
// Host pointers are fake addresses, compared and never dereferenced.
#include "lema_slot.cpp"

#include <cstdio>
#include <random>

namespace {

int fail(const char *what, int trial) {
    std::printf("FAIL trial %d: %s\n", trial, what);
    return 1;
}

}  // namespace

int main() {
    std::mt19937_64 rng(20261202);
    long pieces = 0;
    for (int trial = 0; trial < 4000; ++trial) {
        LayerPlan plan;
        PlanBuilder b{&plan};
        const uintptr_t host0 = uintptr_t(1) << 40;
        size_t hoff = 0;
        const int n = 1 + int(rng() % 12);
        for (int i = 0; i < n; ++i) {
            size_t bytes;
            switch (rng() % 6) {
            case 0: bytes = rng() % 1000; break;                                   // tiny, or empty
            case 1: bytes = rng() % (size_t(1) << 20); break;
            case 2: bytes = kStageChunk - 256 * (rng() % 3) + rng() % 3; break;   // about one chunk
            case 3: bytes = (rng() % 3 + 1) * kStageChunk + rng() % 5000; break;  // several chunks
            case 4: bytes = 4 * (rng() % 4096); break;                            // row scales
            default: bytes = rng() % (size_t(300) << 20);
            }
            const int dir = int(rng() % 3);                                       // in+out, in, out
            b.add(reinterpret_cast<void *>(host0 + hoff), bytes, dir != 2, dir != 1);
            hoff += bytes + 4096;
        }
        for (int inbound = 0; inbound < 2; ++inbound) {
            auto mine = [&](const Xfer &x) { return x.bytes > 0 && (inbound ? x.in : x.out); };
            auto other = [&](const Xfer &x) { return x.bytes > 0 && !(inbound ? x.in : x.out); };
            std::vector<Piece> ps;
            plan_pieces(plan, inbound != 0, &ps);
            std::vector<std::pair<size_t, size_t>> got;   // slot offset, bytes of each part
            for (const Piece &p : ps) {
                if (p.span == 0 || p.span > kStageChunk || p.parts.empty()) return fail("span", trial);
                if (p.slot_off % kSlotAlign != 0) return fail("alignment", trial);
                size_t end = 0;
                for (const PiecePart &q : p.parts) {
                    if (q.bytes == 0 || q.at < end || q.at + q.bytes > p.span) return fail("part order", trial);
                    end = q.at + q.bytes;
                    const size_t so = p.slot_off + q.at;
                    bool found = false;
                    for (const Xfer &x : plan.xfers) {
                        if (!mine(x) || so < x.off || so + q.bytes > x.off + x.bytes) continue;
                        if (q.host != x.host + (so - x.off)) return fail("host address", trial);
                        found = true;
                    }
                    if (!found) return fail("part outside the direction's arrays", trial);
                    got.push_back({so, q.bytes});
                }
                if (end != p.span) return fail("span end", trial);
                for (const Xfer &x : plan.xfers)
                    if (other(x) && x.off < p.slot_off + p.span && x.off + x.bytes > p.slot_off)
                        return fail("other direction inside a span", trial);
            }
            std::sort(got.begin(), got.end());
            size_t gi = 0;
            for (const Xfer &x : plan.xfers) {
                if (!mine(x)) continue;
                size_t pos = x.off;
                while (gi < got.size() && got[gi].first == pos && pos < x.off + x.bytes)
                    pos += got[gi++].second;
                if (pos != x.off + x.bytes) return fail("coverage", trial);
            }
            if (gi != got.size()) return fail("parts beyond the arrays", trial);
            pieces += long(ps.size());
        }
    }
    std::printf("ok %ld pieces\n", pieces);
    return 0;
}
