// Host check of the decode kernels' per-segment address arithmetic
// (segment_plan.h, compiled here for the CPU exactly as the kernels use it).
//
// A segment's writes depend only on its two segment records (g0 = its first
// element, g1 = the next segment's) and the view's sizes, never on the
// exponent stream ([P3] "DFloat11重新定义LLM无损压缩的技术边界" 2.2: the
// reconstruct phase writes at positions given by the prefix sum, which here
// add up to g1 - g0 or the segment is skipped).  For random and corrupt
// records this program checks, for every lane:
//   - an inconsistent segment (g1 < g0, g1 > n, or too large for the
//     staging) plans no unit and is skipped;
//   - otherwise every 16-byte unit store, every ragged one-element store,
//     every staging read and every sign+mantissa load lies inside its
//     array, and the stores cover the segment's elements exactly once
//     (row-major, the fused kernel's tile order written row-major, and a
//     row of an embedding gather).
// Exit status 0 and "ok" when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../segment_plan.h"

using namespace df11plan;

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t rnd()
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}
uint64_t rnd_below(uint64_t m) { return m ? rnd() % m : 0; }

long g_checks = 0, g_fail = 0;
void expect(bool ok, const char *what, uint64_t a, uint64_t b, uint64_t c)
{
    g_checks++;
    if (!ok && g_fail++ < 20) std::printf("FAIL %s (%llu %llu %llu)\n", what, (unsigned long long)a, (unsigned long long)b,
                                          (unsigned long long)c);
}

// rounds of units whose sign+mantissa bytes are loaded before the decode:
// 6 or 5 by chunk size and store mode, both checked
int g_prefetch = 5;

// Row-major merge of elements [lo, hi) of a plan (merge_range): unit
// stores, ragged stores, staging reads, sign+mantissa loads.  cover[g - lo]
// counts the stores of element g when cover is given.
void check_range(const SegPlan &p, uint64_t lo, uint64_t hi, uint64_t n, uint64_t n_sm, uint32_t stg_bytes,
                 std::vector<uint8_t> *cover)
{
    // sign+mantissa prefetch: lanes past the last unit reload the last one
    const uint32_t last = p.nunits ? p.nunits - 1 : 0u;
    const uint64_t base = p.nunits ? p.gbase : 0ull;
    for (uint32_t lane = 0; lane < 64; lane++)
        for (int r = 0; r < g_prefetch; r++) {
            const uint64_t u = std::min<uint64_t>(lane + 64u * r, last);
            expect(base + 8 * u + 8 <= n_sm, "prefetch load inside sm", base, u, n_sm);
        }
    if (!p.valid) return;
    for (uint32_t ui = 0; ui < p.nunits; ui++) {
        expect(p.gbase + 8ull * ui + 8 <= n_sm, "unit load inside sm", p.gbase, ui, n_sm);
        if (!unit_inside(p, lo, hi, ui)) continue;
        const uint64_t gs = p.gbase + 8ull * ui;
        expect(gs + 8 <= n, "unit store inside out", gs, n, 0);
        expect(8ull * ui + 8 <= stg_bytes, "unit staging read inside staging", ui, stg_bytes, 0);
        if (cover)
            for (int e = 0; e < 8; e++) (*cover)[gs + e - lo]++;
    }
    for (uint32_t lane = 0; lane < 64; lane++) {
        const RaggedLane rg = ragged_lane(lo, hi, lane);
        if (!rg.act) continue;
        expect(rg.g >= lo && rg.g < hi && rg.g < n, "ragged store inside range", rg.g, lo, hi);
        expect(rg.g - p.gbase < stg_bytes, "ragged staging read inside staging", rg.g, p.gbase, stg_bytes);
        if (cover) (*cover)[rg.g - lo]++;
    }
}

void check_cover(const std::vector<uint8_t> &cover, const char *what, uint64_t a, uint64_t b)
{
    for (size_t i = 0; i < cover.size(); i++)
        if (cover[i] != 1) {
            expect(false, what, a, b, i);
            return;
        }
    expect(true, what, a, b, 0);
}

// records: random, or corrupt (reversed, past n, huge)
void row_major_cases(long iters)
{
    for (long it = 0; it < iters; it++) {
        const uint64_t n = (it % 3 == 0) ? rnd_below(1ull << 40) : rnd_below(200000) + 1;
        const uint64_t n_sm = (n + 15) / 16 * 16;
        const uint32_t stg = (uint32_t)((rnd_below(65520 - 64) + 64) & ~15u);
        uint64_t g0, g1;
        switch (rnd_below(5)) {
        case 0: g0 = rnd(); g1 = rnd(); break;                                   // garbage
        case 1: g0 = rnd_below(n + 1); g1 = g0 - rnd_below(9000) - 1; break;     // reversed
        case 2: g0 = rnd_below(n + 1); g1 = n + rnd_below(9000) + 1; break;      // past n
        default: g0 = rnd_below(n + 1); g1 = std::min(n, g0 + rnd_below(12000)); break;   // plausible
        }
        const SegPlan p = plan_segment(g0, g1, n, stg);
        const bool ok = g1 >= g0 && g1 <= n && (g0 & 7) + (g1 - g0) + 32 <= stg;
        expect(p.valid == ok, "plan valid exactly when consistent and fitting", g0, g1, n);
        if (!p.valid) expect(p.nunits == 0, "invalid plan has no units", g0, g1, 0);
        // the emit writes codes [head + excl, head + excl + count) of the
        // staging, the counts adding up to g1 - g0
        if (p.valid) expect(p.head + (g1 - g0) <= stg, "emit inside staging", p.head, g1 - g0, stg);
        std::vector<uint8_t> cover;
        const bool small = p.valid && g1 - g0 <= 20000;
        if (small) cover.assign(g1 - g0, 0);
        check_range(p, g0, g1, n, n_sm, stg, small ? &cover : nullptr);
        if (small) check_cover(cover, "row-major stores cover the segment once", g0, g1);
    }
}

// rows of an embedding gather: [lo, hi) = one row, intersected with the segment
void row_gather_cases(long iters)
{
    for (long it = 0; it < iters; it++) {
        const uint64_t cols = 8 * (rnd_below(2000) + 1), nrows = rnd_below(300) + 1, n = cols * nrows;
        const uint64_t n_sm = (n + 15) / 16 * 16;
        const uint32_t stg = (uint32_t)((rnd_below(65520 - 64) + 64) & ~15u);
        const uint64_t g0 = rnd_below(n + 1), g1 = std::min(n, g0 + rnd_below(12000));
        const uint64_t r = rnd_below(nrows), lo = r * cols, hi = lo + cols;
        const SegPlan p = plan_segment(g0, g1, n, stg);
        const uint64_t mlo = std::max(lo, p.g0), mhi = std::min(hi, p.g1);
        if (!p.valid || mlo >= mhi) continue;
        std::vector<uint8_t> cover(mhi - mlo, 0);
        check_range(p, mlo, mhi, n, n_sm, stg, &cover);
        for (uint64_t g = mlo; g < mhi; g++) expect(g - lo < cols, "gather store inside the output row", g, lo, cols);
        check_cover(cover, "gather stores cover the row's part of the segment once", mlo, mhi);
    }
}

// the row gather's window kernel: the row's sign+mantissa bytes in LDS
// (row_bytes = cols rounded up to 16), read at g - lo for every element the
// merge writes, and the output row written at g - lo; a window segment is
// merged only when it overlaps the row and its plan is valid
void row_window_cases(long iters)
{
    for (long it = 0; it < iters; it++) {
        const uint64_t cols = 8 * (rnd_below(4096) + 1), nrows = rnd_below(300) + 1, n = cols * nrows;
        const uint64_t row_bytes = (cols + 15) & ~15ull;
        const uint32_t stg = (uint32_t)((rnd_below(65520 - 64) + 64) & ~15u);
        uint64_t g0, g1;
        switch (rnd_below(4)) {
        case 0: g0 = rnd(); g1 = rnd(); break;                                 // garbage
        case 1: g0 = rnd_below(n + 1); g1 = g0 - rnd_below(9000) - 1; break;   // reversed
        default: g0 = rnd_below(n + 1); g1 = std::min(n, g0 + rnd_below(12000)); break;
        }
        const uint64_t r = rnd_below(nrows), lo = r * cols, hi = lo + cols;
        if (g0 >= hi || g1 <= lo) continue;   // not merged
        const SegPlan p = plan_segment(g0, g1, n, stg);
        if (!p.valid) continue;
        const uint64_t mlo = std::max(lo, p.g0), mhi = std::min(hi, p.g1);
        std::vector<uint8_t> cover(mhi > mlo ? mhi - mlo : 0, 0);
        for (uint32_t ui = 0; ui < p.nunits; ui++) {
            if (!unit_inside(p, mlo, mhi, ui)) continue;
            const uint64_t gs = p.gbase + 8ull * ui;
            expect(gs >= lo && gs - lo + 8 <= cols, "window unit inside the output row", gs, lo, cols);
            expect(gs - lo + 8 <= row_bytes, "window unit's bytes inside the LDS row copy", gs, lo, row_bytes);
            expect(8ull * ui + 8 <= stg, "window unit staging read inside staging", ui, stg, 0);
            for (int e = 0; e < 8; e++) cover[gs + e - mlo]++;
        }
        for (uint32_t lane = 0; lane < 64; lane++) {
            const RaggedLane rg = ragged_lane(mlo, mhi, lane);
            if (!rg.act) continue;
            expect(rg.g >= lo && rg.g - lo < cols, "window ragged store inside the output row", rg.g, lo, cols);
            expect(rg.g - p.gbase < stg, "window ragged staging read inside staging", rg.g, p.gbase, stg);
            cover[rg.g - mlo]++;
        }
        check_cover(cover, "window stores cover the row's part of the segment once", mlo, mhi);
    }
}

// the fused kernel's order: 32-row tiles of 2^tcs columns in 8-column groups,
// a segment inside one tile written row-major (merge_tile_groups8)
void tile_cases(long iters)
{
    for (long it = 0; it < iters; it++) {
        const uint32_t tcs = 4 + (uint32_t)rnd_below(6);            // 16 .. 512 columns
        const uint64_t tc = 1ull << tcs, tpr = rnd_below(8) + 1, rb = rnd_below(6) + 1;
        const uint64_t cols = tc * tpr, rows = 32 * rb, n = rows * cols, tile = 32 * tc;
        const uint32_t stg = (uint32_t)((rnd_below(65520 - 64) + 64) & ~15u);
        const uint64_t t = rnd_below(tpr * rb);
        const uint64_t g0 = t * tile + rnd_below(tile), g1 = std::min((t + 1) * tile, g0 + rnd_below(9000) + 1);
        const SegPlan p = plan_segment(g0, g1, n, stg);
        if (!p.valid) continue;
        const TileSeg q = tile_seg(p, tcs, (uint32_t)tpr, cols, stg);
        std::vector<uint8_t> cover(g1 - g0, 0);
        auto tile_elem = [&](uint64_t out) {   // output element -> stream element of the tile
            const uint64_t r = out / cols, c = out % cols;
            const uint64_t tr = r / 32, tcb = c / tc, rr = r % 32, cc = c % tc;
            return (tr * tpr + tcb) * tile + (cc / 8) * 256 + rr * 8 + cc % 8;
        };
        for (uint32_t gb = q.grp_a; gb <= q.grp_b; gb += 8)
            for (uint32_t k = 0; k < 4; k++)
                for (uint32_t lane = 0; lane < 64; lane++) {
                    const uint32_t e0 = tile_unit(gb, k, lane);
                    // loads of lanes outside the segment reload its first unit
                    const uint64_t ld = q.sm_off + (tile_unit_in(q, gb, e0, lane) ? e0 : (q.lo & ~7u));
                    expect(ld + 8 <= n, "tile sign+mantissa load inside sm", ld, n, 0);
                    if (!tile_unit_in(q, gb, e0, lane)) continue;
                    // staging byte of the unit (LDS addresses are 32-bit: stg_t may wrap)
                    const uint32_t soff = q.stg_t + e0 - stg;
                    expect((uint64_t)soff + 8 <= stg, "tile staging read inside staging", soff, stg, 0);
                    const uint64_t out = q.out_off + tile_unit_out(gb, k, lane, cols);
                    expect(out + 8 <= n && out % cols + 8 <= cols, "tile store inside out, one row", out, n, cols);
                    for (int e = 0; e < 8; e++) {
                        const uint64_t g = tile_elem(out + e);
                        expect(g == q.sm_off + e0 + e, "tile store holds its own element", g, e0, e);
                        if (g >= g0 && g < g1) cover[g - g0]++;
                    }
                }
        for (uint32_t lane = 0; lane < 64; lane++) {   // ragged ends, one element each
            const RaggedLane rg = ragged_lane(g0, g1, lane);
            if (!rg.act) continue;
            expect(rg.g >= g0 && rg.g < g1, "tile ragged inside segment", rg.g, g0, g1);
            cover[rg.g - g0]++;
        }
        check_cover(cover, "tile stores cover the segment once", g0, g1);
    }
}

}  // namespace

int main(int argc, char **argv)
{
    const long iters = argc > 1 ? std::atol(argv[1]) : 20000;
    if (argc > 2) g_state ^= (uint64_t)std::atoll(argv[2]) * 0x2545F4914F6CDD1Dull;
    row_major_cases(iters);
    row_gather_cases(iters / 4);
    row_window_cases(iters / 4);
    g_prefetch = 6;
    row_major_cases(iters / 4);
    tile_cases(iters / 4);
    std::printf("%s: %ld checks, %ld failed\n", g_fail ? "FAILED" : "ok", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
