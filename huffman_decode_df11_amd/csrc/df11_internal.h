// Internal declarations shared by the host sources of libdf11.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/df11.h"

namespace df11 {

// Record a failure for df11_last_error() and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

void canonical_codes(const uint8_t *len, uint32_t *code);
uint16_t chain_walk(const uint16_t *chain, uint32_t window);
int build_tables(df11_codebook *cb);

// Layout checks shared by the host and device encoders: defaults filled in
// (chunk_bytes 16, seg_lanes 64), then the layout checked against n.
df11_layout complete_layout(const df11_layout *in);
int check_layout(const df11_layout &L, uint64_t n);
// A chunk's code count is stored in a byte: chunk bits / shortest code <= 255.
int check_counts_fit(const df11_layout &L, const df11_codebook *cb);

// Compute units of the current device (queried once per device).
int cu_count();

// The row window of a row-major [rows, cols] encoding (df11_view
// row_win_lo / row_win_span) from its n_segments + 1 segment records:
// g(r) = floor((double)(r * cols) * ((double)n_segments / n)); lo = the
// least (first segment of row r) - g(r) and span = the largest (last
// segment of row r) - g(r) - lo + 1 over all rows.  (0, 0) when rows or
// cols is 0, the layout is tiled, or the window does not fit the fields.
void row_window(const df11_segment *segs, uint64_t n_segments, uint64_t n, const df11_layout &L, int32_t *lo,
                uint32_t *span);

}  // namespace df11

struct df11_encoded {
    uint64_t n = 0, total_bits = 0, n_segments = 0;
    df11_layout layout{};
    uint32_t min_len = 0, max_len = 0, n_tables = 0, fast_bits = 0, max_seg_elems = 0;
    int32_t row_win_lo = 0;
    uint32_t row_win_span = 0;
    std::vector<uint32_t> exp_words;
    std::vector<uint8_t> sm;
    std::vector<uint8_t> gaps;
    std::vector<df11_segment> segs;
    std::vector<uint16_t> chain;
    std::vector<uint32_t> fast;
    std::vector<uint64_t> block_seg;
    std::vector<uint8_t> counts;
};
